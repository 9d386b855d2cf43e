// C ABI of the KDA operator: argument validation and kernel launches.
// Everything here runs on the host; nothing is enqueued unless every check
// passes.  See include/kda.h for the contract.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_launch.h"


namespace {

constexpr int64_t kHeadDim = 128;
constexpr int32_t kOrderMax = 4096;       // sequences sorted longest-first up to this count
constexpr int64_t kMaxGrid = 0x7fffffffLL;
constexpr int64_t kChunk = 32;             // tokens per chunk inside the kernel
constexpr int64_t kMinSegTokens = 2048;    // shortest segment worth a separate chain
constexpr int64_t kStateBytes = kHeadDim * kHeadDim * 4;
constexpr int64_t kFillUnits = 256;        // compute units to cover
constexpr int32_t kMaxRecurrent = 64;      // tokens per request on the recurrent path
// floats per (chunk, head) of the backward's chunk matrices: T^T, M^T, P
// [32][32] each, K_end^T, Q+^T, -(B_beta K+)^T [128][32] each, e^{g_C} [128]
constexpr int64_t kBwdChunkElems = 3 * 32 * 32 + 3 * 128 * 32 + 128;

// Sequence-parallel split of an equal-length batch.  Every sequence is cut
// into P segments: segment 0, P - 2 middle segments of L tokens and the last
// segment.  Pass 1: segment 0 starts from the known initial state, so it
// runs once, writing o, on the two-slice kernel (two workgroups per
// (sequence, head)), beside the dual-chain pass over the middle segments
// (one workgroup each; zero start and identity start on the same tiles).
// The merge gives the incoming state of every later segment.  Pass 2: the
// middle segments rerun from theirs on the one-slice kernel (one workgroup
// each), beside the last segment, which has no dual pass and runs once on
// the two-slice kernel.  Each pass holds units * P workgroups, within the
// 256 compute units.  The two-slice chains step through a chunk faster than
// the others, so segment 0 and the last segment are made longer than L by
// the ratios (in sixteenths, per input type) that ran the 1M-token, 16-head
// shape fastest: bf16 34 and 26 (16.07 ms, against 16.36 with the last
// segment as long as the middle ones and rerun beside them, and 17.5 with
// every segment through the dual pass; 18 and 34 for the last one gave
// 16.38 and 17.34), fp32 32 and 28 (262,144 tokens: 9.28 ms against 9.49
// and 10.09; 20 and 32 gave 9.39 and 9.74).
struct Split {
    int32_t P;       // segments per sequence (1: no split)
    int64_t L;       // tokens of every middle segment
    int64_t first;   // tokens of segment 0 (the last one has the rest)
};

// Segments per sequence; the workspace depends on this count only.
int32_t seg_count(int64_t n_seqs, int64_t T, int64_t H) {
    const int64_t units = n_seqs * H;
    if (units <= 0 || T <= 0 || units * 4 > kFillUnits) return 1;
    int64_t P = kFillUnits / units;
    const int64_t by_len = T / kMinSegTokens;
    if (P > by_len) P = by_len;
    return P < 3 ? 1 : (int32_t)P;
}

// Segment 0 : L = R0 / 16 and last : L = R1 / 16.  With T >= 2048 P and
// ratios of 16 .. 48 sixteenths, L (rounded down to whole chunks) and
// segment 0 come to at least 864 tokens and the last segment to at least
// 832: the plan never degenerates (the check below only guards the
// arithmetic).
Split split_for(int64_t n_seqs, int64_t T, int64_t H, bool bf16_in) {
    const int64_t R0 = bf16_in ? 34 : 32;
    const int64_t R1 = bf16_in ? 26 : 28;
    const int64_t P = seg_count(n_seqs, T, H);
    if (P < 3) return Split{1, T, T};
    const int64_t L = 16 * T / (16 * (P - 2) + R0 + R1) / kChunk * kChunk;
    const int64_t first = (R0 * L / 16 + kChunk - 1) / kChunk * kChunk;
    if (L < kChunk || first < kChunk || T - first - (P - 2) * L < kChunk) return Split{1, T, T};
    return Split{(int32_t)P, L, first};
}

// A second stream per device (default priority, not synchronising with the
// null stream) on which one launch of a pair runs beside the other (the
// backward's chunk-matrix pass beside the forward pass it does not depend
// on; the sequence-parallel prefill's first or last segment beside its
// middle segments), and the two events that order it against the caller's
// stream.  Created on first use and kept until the
// process ends (events are never destroyed while a wait may still refer to
// them); a call holds the device's lock while it enqueues, so calls from
// several host threads cannot interleave their records.
constexpr int kMaxDevices = 64;
struct Side {
    std::mutex mu;
    bool tried = false;
    hipStream_t stream = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
};
Side* side_for(int dev) {
    static Side sides[kMaxDevices];
    return dev >= 0 && dev < kMaxDevices ? &sides[dev] : nullptr;
}

// Fork / join of side-stream passes: fork() makes the side stream wait for
// everything enqueued on `main` so far and returns it; join() makes `main`
// wait for what was enqueued on the side stream since.  Without a side
// stream both are no-ops and the passes run on `main` in order.  A fork
// still open when the call returns (an early error return after a failed
// launch) is joined by the destructor, so work already on the side stream
// is ordered before whatever the caller enqueues on `main` next (freeing
// the workspace, say).
struct Fork {
    hipStream_t main;
    Side* sd = nullptr;
    std::unique_lock<std::mutex> lock;
    bool ok = true;
    bool pending = false;   // side-stream work not yet joined
    explicit Fork(hipStream_t s) : main(s) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) return;
        Side* c = side_for(dev);
        if (!c) return;
        lock = std::unique_lock<std::mutex>(c->mu);
        if (!c->tried) {
            c->tried = true;
            if (hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking) != hipSuccess ||
                hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming) != hipSuccess ||
                hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming) != hipSuccess)
                c->stream = nullptr;   // (a partly created set is simply not used)
        }
        if (c->stream) sd = c;
    }
    hipStream_t fork() {
        if (!sd) return main;
        if (hipEventRecord(sd->ev_fork, main) != hipSuccess || hipStreamWaitEvent(sd->stream, sd->ev_fork, 0) != hipSuccess)
            ok = false;
        pending = true;
        return sd->stream;
    }
    void join() {
        if (!sd) return;
        pending = false;
        if (hipEventRecord(sd->ev_join, sd->stream) != hipSuccess || hipStreamWaitEvent(main, sd->ev_join, 0) != hipSuccess)
            ok = false;
    }
    ~Fork() {
        if (pending) join();
    }
    Fork(const Fork&) = delete;
    Fork& operator=(const Fork&) = delete;
};

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t bytes) {
    uintptr_t a = (uintptr_t)p;
    return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlaps(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

int64_t elem_size(int dtype) { return dtype == KDA_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_str(int status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL_POINTER: return "KDA_ERR_NULL_POINTER: a required pointer is NULL";
        case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE: dk/dv must be 128, sizes non-negative, H >= 1";
        case KDA_ERR_BAD_DTYPE: return "KDA_ERR_BAD_DTYPE: in_dtype must be KDA_BF16 or KDA_F32";
        case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED: tensors need 16-byte alignment (beta, cu_seqlens 4-byte)";
        case KDA_ERR_ALIASING: return "KDA_ERR_ALIASING: an output overlaps an input";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_TOO_LARGE: return "KDA_ERR_TOO_LARGE: sizes exceed the launch limits (or H > KDA_MAX_HEADS)";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: kernel launch failed";
        default: return "unknown kda_status";
    }
}

size_t kda_chunk_fwd_workspace_bytes(int32_t n_seqs, int64_t T, int32_t H, int32_t dk,
                                     int32_t dv, int varlen) {
    if (n_seqs < 0 || dk != kHeadDim || dv != kHeadDim || H < 1 || T < 0) return 0;
    if (H > KDA_MAX_HEADS) return 0;
    if (varlen) return n_seqs > kOrderMax ? 0 : (size_t)n_seqs * sizeof(int32_t);
    const int32_t P = seg_count(n_seqs, T, H);
    if (P < 3) return 0;
    // transitions and zero-start final states of the P - 2 middle segments,
    // incoming states of the P - 1 later segments, segment 0's final state
    return (size_t)(3 * P - 4) * n_seqs * H * kStateBytes;
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, int in_dtype,
                  const float* log_alpha, const float* beta, const float* S0,
                  const int32_t* cu_seqlens, int32_t n_seqs, int64_t T, int32_t H, int32_t dk,
                  int32_t dv, float* o, float* S_T, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32) return KDA_ERR_BAD_DTYPE;
    if (dk != kHeadDim || dv != kHeadDim || H < 1 || n_seqs < 0 || T < 0)
        return KDA_ERR_BAD_SHAPE;
    if (H > KDA_MAX_HEADS) return KDA_ERR_TOO_LARGE;
    const bool varlen = cu_seqlens != nullptr;
    int64_t tokens = 0;  // rows of the token axis
    if (varlen) {
        tokens = T;
    } else if (!mul_ok((int64_t)n_seqs, T, &tokens)) {
        return KDA_ERR_TOO_LARGE;
    }
    if (n_seqs == 0) return KDA_OK;
    int64_t rows = 0, elems = 0;
    if (!mul_ok(tokens, (int64_t)H, &rows) || !mul_ok(rows, kHeadDim, &elems) ||
        elems > INT64_MAX / 8)
        return KDA_ERR_TOO_LARGE;
    int64_t units = 0, st_elems = 0;
    if (!mul_ok((int64_t)n_seqs, (int64_t)H, &units) ||
        !mul_ok(units, kHeadDim * kHeadDim, &st_elems))
        return KDA_ERR_TOO_LARGE;
    if (units > INT32_MAX) return KDA_ERR_TOO_LARGE;

    if (tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_NULL_POINTER;

    const int64_t es = elem_size(in_dtype);
    if (tokens > 0) {
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(log_alpha, 16) ||
            !aligned(o, 16) || !aligned(beta, 4))
            return KDA_ERR_MISALIGNED;
    }
    if ((S0 && !aligned(S0, 16)) || (S_T && !aligned(S_T, 16)) ||
        (cu_seqlens && !aligned(cu_seqlens, 4)))
        return KDA_ERR_MISALIGNED;

    // Aliasing: o and S_T against every input; S_T may equal S0 exactly.
    const Range rq = span(q, elems * es), rk = span(k, elems * es), rv = span(v, elems * es);
    const Range rla = span(log_alpha, elems * 4), rb = span(beta, rows * 4);
    const Range ro = span(o, elems * 4);
    const Range rs0 = span(S0, S0 ? st_elems * 4 : 0), rst = span(S_T, S_T ? st_elems * 4 : 0);
    const Range rcu = span(cu_seqlens, varlen ? ((int64_t)n_seqs + 1) * 4 : 0);
    const Range ins[] = {rq, rk, rv, rla, rb, rs0, rcu};
    for (const Range& r : ins)
        if (overlaps(ro, r)) return KDA_ERR_ALIASING;
    if (overlaps(ro, rst)) return KDA_ERR_ALIASING;
    const Range ins_no_s0[] = {rq, rk, rv, rla, rb, rcu};
    for (const Range& r : ins_no_s0)
        if (overlaps(rst, r)) return KDA_ERR_ALIASING;
    if (S0 && S_T && S0 != (const float*)S_T && overlaps(rs0, rst)) return KDA_ERR_ALIASING;

    // Packed batches need the order workspace; equal-length batches use the
    // sequence-parallel path only when the caller provides its workspace.
    const size_t need = kda_chunk_fwd_workspace_bytes(n_seqs, T, H, dk, dv, varlen ? 1 : 0);
    bool use_ws = false;
    if (varlen && need > 0) {
        if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return KDA_ERR_MISALIGNED;
        use_ws = true;
    } else if (!varlen && need > 0 && workspace && workspace_bytes >= need) {
        if (!aligned(workspace, 16)) return KDA_ERR_MISALIGNED;
        use_ws = true;
    }
    if (use_ws) {
        const Range rw = span(workspace, (int64_t)need);
        const Range all[] = {rq, rk, rv, rla, rb, rs0, rcu, ro, rst};
        for (const Range& r : all)
            if (overlaps(rw, r)) return KDA_ERR_ALIASING;
    }

    // Two value-column slices per head (16 columns per wave) when there are
    // too few (sequence, head) units to cover the 256 compute units.
    const int n_slices = units < 256 ? 2 : 1;
    const int wcols = 128 / (4 * n_slices);
    const int64_t grid = ((units + 7) / 8) * 8 * n_slices;
    if (grid > kMaxGrid) return KDA_ERR_TOO_LARGE;

    kda::PrefillParams p{};
    p.seg_len = T;
    p.seg_per_seq = 1;
    p.seg_first = 0;
    p.seg_r0 = 0;
    p.seg_sel = -1;
    p.s0_identity = 0;
    p.h_states = nullptr;
    p.r_out = nullptr;
    p.u_out = nullptr;
    p.S_T2 = nullptr;
    p.q = q;
    p.k = k;
    p.v = v;
    p.la = log_alpha;
    p.beta = beta;
    p.S0 = S0;
    p.cu = cu_seqlens;
    p.order = varlen && use_ws ? (const int32_t*)workspace : nullptr;
    p.o = o;
    p.S_T = S_T;
    p.T = T;
    p.n_seqs = n_seqs;
    p.H = H;
    p.n_slices = n_slices;
    p.n_units = (int32_t)units;
    const bool bf16_in = in_dtype == KDA_BF16;
    const Split sp = varlen || !use_ws ? Split{1, T, T} : split_for(n_seqs, T, H, bf16_in);
    if (sp.P < 3) {
        hipError_t e = kda::launch_chunk_fwd(p, bf16_in, wcols, varlen && use_ws, stream);
        return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }

    // Sequence-parallel path (equal lengths, few chains; the plan is
    // described at split_for).  Each pass runs its two launches on the
    // caller's stream and the second stream, joined before what follows.
    const int32_t n_mid = sp.P - 2;
    const int64_t st = kHeadDim * kHeadDim;
    const int64_t mid_units = units * n_mid;
    float* wF = (float*)workspace;             // [n_seqs * n_mid, H] transitions
    float* wSl = wF + mid_units * st;          // [n_seqs * n_mid, H] zero-start final states
    float* wSmid = wSl + mid_units * st;       // [n_seqs * n_mid, H] incoming states
    float* wSlast = wSmid + mid_units * st;    // [n_seqs, H] the last segment's incoming states
    float* wE = wSlast + units * st;           // [n_seqs, H] segment 0's final states
    if (2 * units + 8 > kMaxGrid || mid_units + 8 > kMaxGrid) return KDA_ERR_TOO_LARGE;

    kda::PrefillParams ps = p;
    ps.seg_len = sp.L;
    ps.seg_first = sp.first;
    kda::PrefillParams p0 = ps;   // segment 0: from S0, writes o and its final state
    p0.seg_len = sp.first;        // (one uniform segment of that length per sequence)
    p0.seg_first = 0;
    p0.seg_per_seq = 1;
    p0.seg_r0 = 0;
    p0.S_T = wE;
    kda::PrefillParams pd = ps;   // middle segments: zero start -> Sl, identity start -> F
    pd.seg_per_seq = n_mid;
    pd.seg_r0 = 1;
    pd.n_seqs = n_seqs * n_mid;
    pd.n_units = (int32_t)mid_units;
    pd.n_slices = 1;
    pd.S0 = nullptr;
    pd.o = nullptr;
    pd.S_T = wSl;
    pd.S_T2 = wF;
    kda::PrefillParams pm = pd;   // middle segments from their incoming states, write o
    pm.S0 = wSmid;
    pm.o = o;
    pm.S_T = nullptr;
    pm.S_T2 = nullptr;
    kda::PrefillParams pl = ps;   // the last segment from its incoming state: o and S_T
    pl.seg_first = sp.first + n_mid * sp.L;   // (everything before it as segment 0)
    pl.seg_len = T;
    pl.seg_per_seq = 1;
    pl.seg_r0 = 1;
    pl.S0 = wSlast;

    Fork fk(stream);
    if (kda::launch_chunk_fwd(p0, bf16_in, 16, false, fk.fork()) != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_chunk_fwd_dual(pd, bf16_in, stream) != hipSuccess) return KDA_ERR_HIP;
    fk.join();
    if (kda::launch_segment_merge(wF, wSl, wE, wSmid, wSlast, n_seqs, n_mid, H, stream) != hipSuccess)
        return KDA_ERR_HIP;
    if (kda::launch_chunk_fwd(pl, bf16_in, 16, false, fk.fork()) != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_chunk_fwd(pm, bf16_in, 32, false, stream) != hipSuccess) return KDA_ERR_HIP;
    fk.join();
    return fk.ok ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_step(const void* q, const void* k, const void* v, int in_dtype,
                    const float* log_alpha, const float* beta, float* S, int32_t B, int32_t H,
                    int32_t dk, int32_t dv, float* o, hipStream_t stream) {
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32) return KDA_ERR_BAD_DTYPE;
    if (dk != kHeadDim || dv != kHeadDim || H < 1 || B < 0) return KDA_ERR_BAD_SHAPE;
    if (H > KDA_MAX_HEADS) return KDA_ERR_TOO_LARGE;
    if (B == 0) return KDA_OK;
    const int64_t states = (int64_t)B * H;
    if (states > kMaxGrid) return KDA_ERR_TOO_LARGE;
    if (!q || !k || !v || !log_alpha || !beta || !S || !o) return KDA_ERR_NULL_POINTER;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(log_alpha, 16) ||
        !aligned(S, 16) || !aligned(o, 16) || !aligned(beta, 4))
        return KDA_ERR_MISALIGNED;
    const int64_t es = elem_size(in_dtype);
    const int64_t elems = states * kHeadDim;
    const Range rq = span(q, elems * es), rk = span(k, elems * es), rv = span(v, elems * es);
    const Range rla = span(log_alpha, elems * 4), rb = span(beta, states * 4);
    const Range rs = span(S, states * kHeadDim * kHeadDim * 4), ro = span(o, elems * 4);
    const Range ins[] = {rq, rk, rv, rla, rb};
    for (const Range& r : ins)
        if (overlaps(ro, r) || overlaps(rs, r)) return KDA_ERR_ALIASING;
    if (overlaps(ro, rs)) return KDA_ERR_ALIASING;
    // one token per request on the recurrent kernel: no replay, state committed
    hipError_t e = kda::launch_recurrent(q, k, v, in_dtype == KDA_BF16, log_alpha, beta, nullptr,
                                         nullptr, nullptr, nullptr, nullptr, nullptr, S, states, H,
                                         1, 0, 1, o, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_recurrent_fwd(const void* q, const void* k, const void* v, int in_dtype,
                      const float* log_alpha, const float* beta, const void* rq,
                      const void* rk, const void* rv, const float* rlog_alpha,
                      const float* rbeta, const int32_t* n_replay, float* S, int32_t B,
                      int32_t T, int32_t Tr, int32_t H, int32_t dk, int32_t dv, int commit,
                      float* o, hipStream_t stream) {
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32) return KDA_ERR_BAD_DTYPE;
    if (dk != kHeadDim || dv != kHeadDim || H < 1 || B < 0 || T < 0 || T > kMaxRecurrent ||
        Tr < 0 || Tr > kMaxRecurrent)
        return KDA_ERR_BAD_SHAPE;
    if (H > KDA_MAX_HEADS) return KDA_ERR_TOO_LARGE;
    if (B == 0) return KDA_OK;
    const int64_t states = (int64_t)B * H;
    if (states > kMaxGrid) return KDA_ERR_TOO_LARGE;
    if (!S) return KDA_ERR_NULL_POINTER;
    if (T > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_NULL_POINTER;
    if (Tr > 0 && (!rq || !rk || !rv || !rlog_alpha || !rbeta)) return KDA_ERR_NULL_POINTER;
    if (!aligned(S, 16)) return KDA_ERR_MISALIGNED;
    if (T > 0 && (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
                  !aligned(log_alpha, 16) || !aligned(o, 16) || !aligned(beta, 4)))
        return KDA_ERR_MISALIGNED;
    if (Tr > 0 && (!aligned(rq, 16) || !aligned(rk, 16) || !aligned(rv, 16) ||
                   !aligned(rlog_alpha, 16) || !aligned(rbeta, 4)))
        return KDA_ERR_MISALIGNED;
    if (n_replay && !aligned(n_replay, 4)) return KDA_ERR_MISALIGNED;
    const int64_t es = elem_size(in_dtype);
    const int64_t e_new = states * T * kHeadDim, e_rep = states * Tr * kHeadDim;
    const Range rs = span(S, states * kHeadDim * kHeadDim * 4);
    const Range ro = span(o, T > 0 ? e_new * 4 : 0);
    const Range ins[] = {span(q, T > 0 ? e_new * es : 0), span(k, T > 0 ? e_new * es : 0),
                         span(v, T > 0 ? e_new * es : 0), span(log_alpha, T > 0 ? e_new * 4 : 0),
                         span(beta, T > 0 ? states * T * 4 : 0),
                         span(rq, Tr > 0 ? e_rep * es : 0), span(rk, Tr > 0 ? e_rep * es : 0),
                         span(rv, Tr > 0 ? e_rep * es : 0),
                         span(rlog_alpha, Tr > 0 ? e_rep * 4 : 0),
                         span(rbeta, Tr > 0 ? states * Tr * 4 : 0),
                         span(n_replay, Tr > 0 && n_replay ? (int64_t)B * 4 : 0)};
    for (const Range& r : ins)
        if (overlaps(ro, r) || overlaps(rs, r)) return KDA_ERR_ALIASING;
    if (overlaps(ro, rs)) return KDA_ERR_ALIASING;
    hipError_t e = kda::launch_recurrent(q, k, v, in_dtype == KDA_BF16, log_alpha, beta, rq, rk,
                                         rv, rlog_alpha, rbeta, Tr > 0 ? n_replay : nullptr, S,
                                         states, H, T, Tr, commit ? 1 : 0, o, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_prologue(const void* q_raw, const void* k_raw, const void* v_raw, int in_dtype,
                 const float* conv_w, float* conv_cache, const float* a, const float* b,
                 const int32_t* cu_seqlens, int32_t n_seqs, int64_t T, int32_t H, int32_t dk,
                 void* q, void* k, void* v, float* log_alpha, float* beta,
                 hipStream_t stream) {
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32) return KDA_ERR_BAD_DTYPE;
    if (dk != kHeadDim || H < 1 || n_seqs < 0 || T < 0) return KDA_ERR_BAD_SHAPE;
    if (H > KDA_MAX_HEADS) return KDA_ERR_TOO_LARGE;
    const bool varlen = cu_seqlens != nullptr;
    int64_t rows = 0, elems = 0, hrows = 0;
    if (varlen) rows = T;
    else if (!mul_ok((int64_t)n_seqs, T, &rows)) return KDA_ERR_TOO_LARGE;
    if (n_seqs == 0) return KDA_OK;
    if (!mul_ok(rows, (int64_t)H, &hrows) || !mul_ok(hrows, kHeadDim, &elems) ||
        elems > INT64_MAX / 8 || ((rows + 7) / 8) * ((H + 3) / 4) > kMaxGrid)
        return KDA_ERR_TOO_LARGE;
    const int64_t cache_elems = (int64_t)n_seqs * 9 * H * kHeadDim;
    if (conv_cache && (cache_elems + 255) / 256 > kMaxGrid) return KDA_ERR_TOO_LARGE;
    if (rows > 0 && (!q_raw || !k_raw || !v_raw || !conv_w || !a || !b || !q || !k || !v ||
                     !log_alpha || !beta))
        return KDA_ERR_NULL_POINTER;
    if (rows > 0 && (!aligned(q_raw, 16) || !aligned(k_raw, 16) || !aligned(v_raw, 16) ||
                     !aligned(conv_w, 16) || !aligned(a, 16) || !aligned(q, 16) ||
                     !aligned(k, 16) || !aligned(v, 16) || !aligned(log_alpha, 16) ||
                     !aligned(b, 4) || !aligned(beta, 4)))
        return KDA_ERR_MISALIGNED;
    if ((conv_cache && !aligned(conv_cache, 16)) || (cu_seqlens && !aligned(cu_seqlens, 4)))
        return KDA_ERR_MISALIGNED;
    const int64_t es = elem_size(in_dtype);
    const Range ins[] = {span(q_raw, elems * es), span(k_raw, elems * es), span(v_raw, elems * es),
                         span(conv_w, rows > 0 ? 3 * (int64_t)H * kHeadDim * 16 : 0),
                         span(a, elems * 4), span(b, hrows * 4),
                         span(cu_seqlens, varlen ? ((int64_t)n_seqs + 1) * 4 : 0)};
    const Range outs[] = {span(q, elems * es), span(k, elems * es), span(v, elems * es),
                          span(log_alpha, elems * 4), span(beta, hrows * 4),
                          span(conv_cache, conv_cache ? cache_elems * 4 : 0)};
    for (int i = 0; i < 6; ++i) {
        for (const Range& r : ins)
            if (overlaps(outs[i], r)) return KDA_ERR_ALIASING;
        for (int j = i + 1; j < 6; ++j)
            if (overlaps(outs[i], outs[j])) return KDA_ERR_ALIASING;
    }
    kda::LayerParams p;
    p.q_raw = q_raw;
    p.k_raw = k_raw;
    p.v_raw = v_raw;
    p.conv_w = conv_w;
    p.cache = conv_cache;
    p.a = a;
    p.b = b;
    p.cu = cu_seqlens;
    p.q = q;
    p.k = k;
    p.v = v;
    p.log_alpha = log_alpha;
    p.beta = beta;
    p.rows = rows;
    p.T = T;
    p.n_seqs = n_seqs;
    p.H = H;
    hipError_t e = kda::launch_prologue(p, in_dtype == KDA_BF16, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_epilogue(const float* o, const float* g, const float* w, int64_t rows, int32_t H,
                 int32_t dv, float* out, hipStream_t stream) {
    if (dv != kHeadDim || H < 1 || rows < 0) return KDA_ERR_BAD_SHAPE;
    if (H > KDA_MAX_HEADS) return KDA_ERR_TOO_LARGE;
    int64_t items = 0, elems = 0;
    if (!mul_ok(rows, (int64_t)H, &items) || !mul_ok(items, kHeadDim, &elems) ||
        elems > INT64_MAX / 8 || (items + 3) / 4 > kMaxGrid)
        return KDA_ERR_TOO_LARGE;
    if (items == 0) return KDA_OK;
    if (!o || !g || !w || !out) return KDA_ERR_NULL_POINTER;
    if (!aligned(o, 16) || !aligned(g, 16) || !aligned(w, 16) || !aligned(out, 16))
        return KDA_ERR_MISALIGNED;
    const Range ro = span(o, elems * 4), rg = span(g, elems * 4), rw = span(w, kHeadDim * 4);
    const Range rout = span(out, elems * 4);
    if (overlaps(rout, rg) || overlaps(rout, rw)) return KDA_ERR_ALIASING;
    if (out != o && overlaps(rout, ro)) return KDA_ERR_ALIASING;
    hipError_t e = kda::launch_epilogue(o, g, w, out, items, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Backward workspace layout (floats): states at chunk starts and gradients
// at chunk ends [slots, H, 128, 128] each, the chunk matrices of the first
// backward pass [slots, H, kBwdChunkElems], and W, V - K+ S and U of every
// token [rows, H, 128] each.  Packed batches: slots = tokens / 32 + n_seqs,
// rows = tokens.  Equal lengths run in windows of W chunks (the last window
// first): slots = n_seqs * W, rows = n_seqs * 32 W, plus the state at the
// start of every window after the first and one state gradient per
// (sequence, head) carried from window to window.
struct BwdLayout {
    int64_t slots, rows, n_win, win_chunks;
    int64_t h, dsn, tmp, w, r, u, ckpt, carry, total;   // offsets and total in floats
};
static bool bwd_layout(int64_t n_seqs, int64_t slots, int64_t rows, int64_t n_win, int64_t H,
                       BwdLayout* L) {
    L->slots = slots;
    L->rows = rows;
    L->n_win = n_win;
    int64_t sh = 0, st = 0, tmp = 0, wv = 0, units = 0, ust = 0, ck = 0;
    if (!mul_ok(slots, H, &sh) || !mul_ok(sh, kHeadDim * kHeadDim, &st) ||
        !mul_ok(sh, kBwdChunkElems, &tmp) || !mul_ok(rows, H * kHeadDim, &wv) ||
        !mul_ok(n_seqs, H, &units) || !mul_ok(units, kHeadDim * kHeadDim, &ust) ||
        !mul_ok(ust, n_win - 1, &ck))
        return false;
    L->h = 0;
    L->dsn = st;
    L->tmp = 2 * st;
    L->w = 2 * st + tmp;
    L->r = L->w + wv;
    L->u = L->r + wv;
    L->ckpt = L->u + wv;
    L->carry = L->ckpt + ck;
    L->total = L->carry + (n_win > 1 ? ust : 0);
    return st <= INT64_MAX / 16 && tmp <= INT64_MAX / 16 && wv <= INT64_MAX / 16 &&
           ck <= INT64_MAX / 16 && L->total >= 0 && L->total <= INT64_MAX / 8;
}
static bool bwd_layout_packed(int64_t n_seqs, int64_t tokens, int64_t H, BwdLayout* L) {
    L->win_chunks = 0;
    return bwd_layout(n_seqs, tokens / kChunk + n_seqs, tokens, 1, H, L);
}
// Equal lengths with windows of W chunks (W >= 1; W >= the chunks of a
// sequence: one window).  At most kMaxBwdWindows windows (five launches
// each): a window so short that more are needed is refused.
constexpr int64_t kMaxBwdWindows = 1 << 16;
static bool bwd_layout_windowed(int64_t n_seqs, int64_t T, int64_t H, int64_t W, BwdLayout* L) {
    const int64_t C = (T + kChunk - 1) / kChunk;
    if (W < 1) return false;
    if (W > C) W = C < 1 ? 1 : C;
    const int64_t n_win = C == 0 ? 1 : (C + W - 1) / W;
    if (n_win > kMaxBwdWindows) return false;
    int64_t slots = 0, rows = 0;
    if (!mul_ok(n_seqs, W, &slots) || !mul_ok(slots, kChunk, &rows)) return false;
    L->win_chunks = W;
    return bwd_layout(n_seqs, slots, rows, n_win, H, L);
}
// The window the backward uses for a workspace of `bytes`: one window if it
// fits, else the longest power-of-two number of chunks that fits.
static bool bwd_pick_window(int64_t n_seqs, int64_t T, int64_t H, size_t bytes, BwdLayout* L) {
    const int64_t C = (T + kChunk - 1) / kChunk;
    if (bwd_layout_windowed(n_seqs, T, H, C < 1 ? 1 : C, L) && (size_t)L->total * 4 <= bytes)
        return true;
    int64_t W = 1;
    while (W * 2 < C) W *= 2;
    for (; W >= 1; W /= 2)
        if (bwd_layout_windowed(n_seqs, T, H, W, L) && (size_t)L->total * 4 <= bytes) return true;
    return false;
}
static int64_t bwd_round_window(int64_t T, int64_t window_tokens) {
    const int64_t C = (T + kChunk - 1) / kChunk;
    const int64_t want = (window_tokens + kChunk - 1) / kChunk;
    if (want >= C) return C < 1 ? 1 : C;
    int64_t W = 1;
    while (W < want) W *= 2;
    return W >= C ? (C < 1 ? 1 : C) : W;
}

size_t kda_chunk_bwd_workspace_bytes_window(int32_t n_seqs, int64_t T, int32_t H, int32_t dk,
                                            int32_t dv, int64_t window_tokens) {
    if (n_seqs < 0 || dk != kHeadDim || dv != kHeadDim || H < 1 || T < 0 || window_tokens < 1)
        return 0;
    if (H > KDA_MAX_HEADS) return 0;
    int64_t tokens = 0;
    if (!mul_ok((int64_t)n_seqs, T, &tokens)) return 0;
    BwdLayout L;
    if (!bwd_layout_windowed(n_seqs, T, H, bwd_round_window(T, window_tokens), &L)) return 0;
    return (size_t)L.total * 4;
}

size_t kda_chunk_bwd_workspace_bytes(int32_t n_seqs, int64_t T, int32_t H, int32_t dk, int32_t dv,
                                     int varlen) {
    if (n_seqs < 0 || dk != kHeadDim || dv != kHeadDim || H < 1 || T < 0) return 0;
    if (H > KDA_MAX_HEADS) return 0;
    if (!varlen) return kda_chunk_bwd_workspace_bytes_window(n_seqs, T, H, dk, dv, KDA_BWD_WINDOW);
    BwdLayout L;
    if (!bwd_layout_packed(n_seqs, T, H, &L)) return 0;
    return (size_t)L.total * 4;
}

int kda_chunk_bwd(const void* q, const void* k, const void* v, int in_dtype,
                  const float* log_alpha, const float* beta, const float* S0,
                  const int32_t* cu_seqlens, int32_t n_seqs, int64_t T, int32_t H, int32_t dk,
                  int32_t dv, const float* grad_o, const float* grad_S_T, float* grad_q,
                  float* grad_k, float* grad_v, float* grad_log_alpha, float* grad_beta,
                  float* grad_S0, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (in_dtype != KDA_BF16 && in_dtype != KDA_F32) return KDA_ERR_BAD_DTYPE;
    if (dk != kHeadDim || dv != kHeadDim || H < 1 || n_seqs < 0 || T < 0)
        return KDA_ERR_BAD_SHAPE;
    if (H > KDA_MAX_HEADS) return KDA_ERR_TOO_LARGE;
    const bool varlen = cu_seqlens != nullptr;
    int64_t tokens = 0;
    if (varlen) tokens = T;
    else if (!mul_ok((int64_t)n_seqs, T, &tokens)) return KDA_ERR_TOO_LARGE;
    if (n_seqs == 0) return KDA_OK;
    int64_t rows = 0, elems = 0, units = 0, st_elems = 0;
    if (!mul_ok(tokens, (int64_t)H, &rows) || !mul_ok(rows, kHeadDim, &elems) ||
        elems > INT64_MAX / 8 || !mul_ok((int64_t)n_seqs, (int64_t)H, &units) ||
        !mul_ok(units, kHeadDim * kHeadDim, &st_elems))
        return KDA_ERR_TOO_LARGE;
    // The largest layout (packed, or one window per sequence) bounds the
    // grids of every layout this call can pick.
    BwdLayout L;
    const bool sizes_ok = varlen ? bwd_layout_packed(n_seqs, tokens, H, &L)
                                 : bwd_layout_windowed(n_seqs, T, H, (T + kChunk - 1) / kChunk + 1, &L);
    if (!sizes_ok) return KDA_ERR_TOO_LARGE;
    if (units > INT32_MAX / 32 || L.slots * H > INT32_MAX) return KDA_ERR_TOO_LARGE;

    if (tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !grad_o || !grad_q || !grad_k ||
                       !grad_v || !grad_log_alpha || !grad_beta))
        return KDA_ERR_NULL_POINTER;
    if (!workspace) return KDA_ERR_WORKSPACE;
    if (varlen ? (size_t)L.total * 4 > workspace_bytes
               : !bwd_pick_window(n_seqs, T, H, workspace_bytes, &L))
        return KDA_ERR_WORKSPACE;
    if (tokens > 0) {
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(log_alpha, 16) ||
            !aligned(grad_o, 16) || !aligned(grad_q, 16) || !aligned(grad_k, 16) ||
            !aligned(grad_v, 16) || !aligned(grad_log_alpha, 16) || !aligned(beta, 4) ||
            !aligned(grad_beta, 4))
            return KDA_ERR_MISALIGNED;
    }
    if ((S0 && !aligned(S0, 16)) || (grad_S_T && !aligned(grad_S_T, 16)) ||
        (grad_S0 && !aligned(grad_S0, 16)) || (cu_seqlens && !aligned(cu_seqlens, 4)) ||
        !aligned(workspace, 16))
        return KDA_ERR_MISALIGNED;

    // Every output (and the workspace) overlaps no input and no other
    // output; grad_S0 may be the same pointer as grad_S_T.
    const int64_t es = elem_size(in_dtype);
    const Range rq = span(q, elems * es), rk = span(k, elems * es), rv = span(v, elems * es);
    const Range rla = span(log_alpha, elems * 4), rb = span(beta, rows * 4);
    const Range rs0 = span(S0, S0 ? st_elems * 4 : 0);
    const Range rcu = span(cu_seqlens, varlen ? ((int64_t)n_seqs + 1) * 4 : 0);
    const Range rgo = span(grad_o, elems * 4);
    const Range rgst = span(grad_S_T, grad_S_T ? st_elems * 4 : 0);
    const Range outs[] = {span(grad_q, elems * 4), span(grad_k, elems * 4), span(grad_v, elems * 4),
                          span(grad_log_alpha, elems * 4), span(grad_beta, rows * 4),
                          span(grad_S0, grad_S0 ? st_elems * 4 : 0),
                          span(workspace, L.total * 4)};
    const Range ins[] = {rq, rk, rv, rla, rb, rs0, rcu, rgo};
    const int n_out = (int)(sizeof(outs) / sizeof(outs[0]));
    for (int a = 0; a < n_out; ++a) {
        for (const Range& r : ins)
            if (overlaps(outs[a], r)) return KDA_ERR_ALIASING;
        const bool gs0 = a == 5;
        if (!(gs0 && grad_S0 == grad_S_T) && overlaps(outs[a], rgst)) return KDA_ERR_ALIASING;
        for (int b = a + 1; b < n_out; ++b)
            if (overlaps(outs[a], outs[b])) return KDA_ERR_ALIASING;
    }

    float* ws = (float*)workspace;
    const bool bf16_in = in_dtype == KDA_BF16;
    const int n_slices = units < 256 ? 2 : 1;
    const int wcols = 128 / (4 * n_slices);
    if (((units + 7) / 8) * 8 * n_slices > kMaxGrid) return KDA_ERR_TOO_LARGE;
    kda::PrefillParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.la = log_alpha;
    p.beta = beta;
    p.S0 = S0;
    p.cu = cu_seqlens;
    p.order = nullptr;
    p.o = nullptr;
    p.S_T = nullptr;
    p.T = T;
    p.seg_len = T;
    p.seg_per_seq = 1;
    p.seg_first = 0;
    p.seg_r0 = 0;
    p.seg_sel = -1;
    p.s0_identity = 0;
    p.n_seqs = n_seqs;
    p.H = H;
    p.n_slices = n_slices;
    p.n_units = (int32_t)units;
    p.h_states = nullptr;
    p.r_out = nullptr;
    p.u_out = nullptr;
    p.S_T2 = nullptr;
    kda::BwdParams b{};
    b.q = q;
    b.k = k;
    b.v = v;
    b.la = log_alpha;
    b.beta = beta;
    b.cu = cu_seqlens;
    b.dO = grad_o;
    b.dS_T = grad_S_T;
    b.dq = grad_q;
    b.dk = grad_k;
    b.dv = grad_v;
    b.dla = grad_log_alpha;
    b.dbeta = grad_beta;
    b.dS0 = grad_S0;
    b.h = ws + L.h;
    b.r = ws + L.r;
    b.u = ws + L.u;
    b.dsn = ws + L.dsn;
    b.tmp = ws + L.tmp;
    b.w = ws + L.w;
    b.T = T;
    b.slots = L.slots;
    b.win_len = 0;
    b.win_idx = 0;
    b.n_seqs = n_seqs;
    b.H = H;
    if (varlen) {
        // 1. forward pass storing the state at every chunk start, V - K+ S
        //    and U; 2. chunk matrices, reverse state-gradient walk, chunk
        //    gradients
        p.h_states = ws + L.h;
        p.r_out = ws + L.r;
        p.u_out = ws + L.u;
        Fork fk(stream);
        if (kda::launch_chunk_bwd_tmp(b, bf16_in, fk.fork()) != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_chunk_fwd(p, bf16_in, wcols, false, stream) != hipSuccess) return KDA_ERR_HIP;
        fk.join();
        if (!fk.ok) return KDA_ERR_HIP;
        return kda::launch_chunk_bwd_walk_grad(b, bf16_in, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    // Equal lengths, windows of W chunks.  The states at the window starts
    // come first (forward passes without per-chunk outputs, window by
    // window); then, from the last window to the first, the forward pass
    // over the window keeping its per-chunk values and the three backward
    // passes, with dL/dS carried from each window to the one before it.
    const int64_t win_len = L.win_chunks * kChunk;
    const int64_t st_el = units * kHeadDim * kHeadDim;
    const int nw = (int)L.n_win;   // <= kMaxBwdWindows
    auto ckpt = [&](int w) -> float* { return w == 0 ? nullptr : ws + L.ckpt + (int64_t)(w - 1) * st_el; };
    p.seg_len = win_len;
    float* carry = nw > 1 ? ws + L.carry : nullptr;
    b.win_len = win_len;
    // The chunk matrices of a window read only the inputs: each runs on the
    // side stream beside the forward pass(es) before its walk, once the
    // previous window's gradients (which read the same workspace) are done.
    Fork fk(stream);
    auto fork_tmp = [&](int w) -> bool {
        kda::BwdParams bw = b;
        bw.win_idx = w;
        return kda::launch_chunk_bwd_tmp(bw, bf16_in, fk.fork()) == hipSuccess;
    };
    if (nw > 0 && !fork_tmp(nw - 1)) return KDA_ERR_HIP;
    for (int w = 0; w + 1 < nw; ++w) {
        kda::PrefillParams pw = p;
        pw.seg_sel = w;
        pw.S0 = w == 0 ? S0 : ckpt(w);
        pw.S_T = ckpt(w + 1);
        if (kda::launch_chunk_fwd(pw, bf16_in, wcols, false, stream) != hipSuccess) return KDA_ERR_HIP;
    }
    for (int w = nw - 1; w >= 0; --w) {
        if (w < nw - 1 && !fork_tmp(w)) return KDA_ERR_HIP;
        kda::PrefillParams pw = p;
        pw.seg_sel = w;
        pw.S0 = w == 0 ? S0 : ckpt(w);
        pw.h_states = ws + L.h;
        pw.r_out = ws + L.r;
        pw.u_out = ws + L.u;
        if (kda::launch_chunk_fwd(pw, bf16_in, wcols, false, stream) != hipSuccess) return KDA_ERR_HIP;
        fk.join();
        kda::BwdParams bw = b;
        bw.win_idx = w;
        bw.dS_T = w == nw - 1 ? grad_S_T : carry;
        bw.dS0 = w == 0 ? grad_S0 : carry;
        if (kda::launch_chunk_bwd_walk_grad(bw, bf16_in, stream) != hipSuccess) return KDA_ERR_HIP;
    }
    return fk.ok ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
