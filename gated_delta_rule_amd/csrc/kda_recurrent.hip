// Multi-token recurrent decode with on-chip replay (gfx950).
//
// Decode with a few tokens per request runs the recurrence token by token
// ("把注意力换成一块「会遗忘的内存」" section "层的实现:低秩门控与两条执行路径":
// sequences of up to 64 tokens take the fused recurrent path, where the
// fixed-size state makes the token loop the fastest form).  For speculative
// decoding, "Kimi K3 技术报告解读" section 9 keeps only the draft tokens'
// inputs and rebuilds the accepted tokens' state on chip, with verification
// and write-back in one kernel.  Both are this kernel: per (request, head)
// the state is loaded once, the first n_replay[b] replay tokens are applied
// (state only), then T tokens are applied with their outputs, and the state
// is stored either after the replay (commit = 0: the T drafts are verified
// but not committed) or after all tokens (commit = 1).
//
// Each token is the three-step update of "Kimi K3 核心算子拆解" section 2.3
// read after the update, in the single-pass form
//   u = beta (v - x),  x = k^T Diag(a) S,  o = y + (q . k) u,  y = q^T Diag(a) S,
//   S <- Diag(a) S + k u^T.
//
// Work decomposition: one workgroup per state at a time; with CPW value
// columns per wave (8: 16 waves, 1024 threads; 16: 8 waves, 512 threads)
// wave w owns columns CPW w .. CPW w + CPW - 1 for all 128 key rows, lane l
// holding column CPW w + (l mod CPW) of rows (l / CPW) + (64 / CPW) i.  The
// sums over key rows then stay inside the wave (cross-lane butterflies, no
// LDS and no barrier per token); waves only share the token data, staged in
// LDS one token per wave at a time.  The state moves between HBM and
// registers through LDS so that both transfers are 1 KB-contiguous per wave
// instruction.  On large batches a workgroup walks up to eight states in
// turn and reads the next state from HBM while it runs the current one's
// last tokens and writes it back, so the state stream does not stop while a
// compute unit computes.  With one or two tokens per state the 1024-thread
// form runs (one workgroup per compute unit streams the state fastest; the
// one-token decode step is this form); with three or more the 512-thread
// form runs, two workgroups per compute unit, so that one's token work
// overlaps the other's state traffic (B=256, H=96: 8 tokens 0.82 against
// 0.91 ms, 64 tokens 3.75 against 4.51, a speculative step of 4 replayed
// and 4 new tokens 0.65 against 0.78; 2 tokens 0.57 against 0.55, hence the
// threshold).  Keeping the 512-thread form's state scaled by the inverse of
// the pass's cumulative decay, so that the decay folds into the staged
// token data (three operations per state element and token instead of
// four), measured no faster (8 tokens 0.81-0.83 ms, 64 tokens 3.82) and is
// not used.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int RC_LDS = 136;      // LDS row stride of the staged state (floats)
constexpr int RC_WIDE_TOKENS = 3;   // tokens per state from which the 512-thread form runs
constexpr int RC_MAX_PER_WG = 8;  // states per workgroup on large batches (measured: 8 ahead of 24, 96, 4, 2, 1)

// x + (value of lane l ^ 8), within each 16-lane row (rotation by 8).
__device__ __forceinline__ float add_xor8(float x) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false));
}
__device__ __forceinline__ float add_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return x + __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return x + __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

struct TokSrc {
    const void* q;
    const void* k;
    const void* v;
    const float* la;
    const float* beta;
    int32_t T;   // tokens per request in this stream
};

template <typename InT, int CPW>
__global__ __launch_bounds__(64 * 128 / CPW, CPW == 16 ? 4 : 1) void recurrent_kernel(TokSrc rep, const int32_t* n_replay,
                                                                   TokSrc out, float* S, float* o,
                                                                   int32_t H, int32_t commit,
                                                                   int64_t n_states, int32_t per_wg) {
    static_assert(CPW == 8 || CPW == 16, "8 or 16 value columns per wave");
    constexpr int RC_THREADS = 64 * 128 / CPW;
    constexpr int RC_TOK = 128 / CPW;          // tokens staged per pass: one per wave
    constexpr int RG = 64 / CPW;               // lane groups: rows rg + RG i
    constexpr int NE = 128 / RG;               // state elements per lane
    constexpr int NPF = 128 * 128 / 4 / RC_THREADS;   // 16-byte state pieces per thread
    constexpr int CSH = CPW == 8 ? 3 : 4, RSH = 6 - CSH;  // log2 CPW, log2 RG
    // The 1024-thread form holds the next state in registers while it runs
    // the current one (it has the compute unit to itself); the 512-thread
    // form reads each state when it starts it and leaves the overlap to the
    // other workgroup on its compute unit (the registers for a read ahead
    // would spill).
    constexpr bool AHEAD = CPW == 8;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & (CPW - 1), rg = lane >> CSH;
    const int col = wave * CPW + c;
    const int64_t first = (int64_t)blockIdx.x * per_wg;
    const int64_t last = first + per_wg < n_states ? first + per_wg : n_states;
    int64_t bh = first, b = 0;
    int h = 0;

    // One LDS area: the staged state while it moves to or from HBM, the token
    // data in between (barriers separate the two uses).  Token data: k, q and
    // the decay factors permuted so that lane group rg reads its rows
    // rg + RG i as NE consecutive floats.
    __shared__ __attribute__((aligned(16))) float smem[128 * RC_LDS];
    float* sS = smem;
    float (*sK)[128] = reinterpret_cast<float (*)[128]>(smem);
    float (*sQ)[128] = reinterpret_cast<float (*)[128]>(smem + RC_TOK * 128);
    float (*sA)[128] = reinterpret_cast<float (*)[128]>(smem + 2 * RC_TOK * 128);
    float (*sV)[128] = reinterpret_cast<float (*)[128]>(smem + 3 * RC_TOK * 128);
    float* sB = smem + 4 * RC_TOK * 128;
    float* sQK = sB + RC_TOK;

    // State reads (the next state's before this state's tokens run, so that
    // it overlaps them, when AHEAD); a state is 1 KB per wave instruction
    // both ways.
    f32x4 pf[NPF];
    auto fetch = [&](int64_t st) {
        const f32x4* g = reinterpret_cast<const f32x4*>(S + st * (128 * 128));
#pragma unroll
        for (int j = 0; j < NPF; ++j) pf[j] = __builtin_nontemporal_load(&g[tid + RC_THREADS * j]);
    };
    // Without a replay stream and with 2..RC_TOK tokens (one staging pass), the
    // next state's token inputs are read ahead too (wave w < T: token w,
    // channels lane and lane + 64), so a state's step starts with no HBM
    // wait (measured on the 1024-thread form with 8 tokens: 0.90 against
    // 0.94 ms at B=256, H=96; with one token
    // it measured slower, 0.540 against 0.511 ms, so it stays off there).
    float tk[2], tq[2], tv[2], tl[2], tb = 0.f;
    bool tok_ready = false;
    const bool tok_ahead = rep.T == 0 && out.T >= 2 && out.T <= RC_TOK;
    auto fetch_tokens = [&](int64_t st) {
        if (wave < out.T) {
            const int64_t sb = st / H;
            const size_t row = ((size_t)sb * out.T + wave) * H + (st - sb * H);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int ch = lane + 64 * half;
                tk[half] = to_f32(((const InT*)out.k)[row * 128 + ch]);
                tq[half] = to_f32(((const InT*)out.q)[row * 128 + ch]);
                tv[half] = to_f32(((const InT*)out.v)[row * 128 + ch]);
                tl[half] = out.la[row * 128 + ch];
            }
            tb = out.beta[row];
        }
        tok_ready = true;
    };
    float s[NE];
    bool fetched = false;
    if constexpr (AHEAD) fetch(first);

    auto store_state = [&]() {
        __syncthreads();   // every lane is done reading sS
#pragma unroll
        for (int i = 0; i < NE; ++i) sS[(rg + RG * i) * RC_LDS + col] = s[i];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int e = tid + RC_THREADS * j;
            __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&sS[(e >> 5) * RC_LDS + 4 * (e & 31)]),
                                        &reinterpret_cast<f32x4*>(S + bh * (128 * 128))[e]);
        }
    };

    // Run n tokens of one stream; outputs when `emit`.
    auto run = [&](const TokSrc& src, int n, bool emit, bool prefetch) {
        for (int t0 = 0; t0 < n; t0 += RC_TOK) {
            const int nt = n - t0 < RC_TOK ? n - t0 : RC_TOK;
            __syncthreads();   // previous tokens consumed
            // stage nt tokens: thread (token tt = tid >> 6, channel pair) -- one wave per token
            if (wave < nt) {
                if (!tok_ready) {   // not read ahead: this pass's tokens now
                    const size_t row = ((size_t)b * src.T + t0 + wave) * H + h;
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int ch = lane + 64 * half;
                        tk[half] = to_f32(((const InT*)src.k)[row * 128 + ch]);
                        tq[half] = to_f32(((const InT*)src.q)[row * 128 + ch]);
                        tv[half] = to_f32(((const InT*)src.v)[row * 128 + ch]);
                        tl[half] = src.la[row * 128 + ch];
                    }
                    tb = src.beta[row];
                }
                float qk = 0.f;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int ch = lane + 64 * half;
                    const int slot = (ch & (RG - 1)) * NE + (ch >> RSH);   // row ch = rg + RG i
                    sK[wave][slot] = tk[half];
                    sQ[wave][slot] = tq[half];
                    sA[wave][slot] = __expf(tl[half]);
                    sV[wave][ch] = tv[half];
                    qk += tq[half] * tk[half];
                }
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) qk += __shfl_xor(qk, off);
                if (lane == 0) {
                    sQK[wave] = qk;
                    sB[wave] = tb;
                }
            }
            tok_ready = false;
            __syncthreads();
            // the next state's read goes out after this pass's last token
            // loads, so that waiting for those does not wait for it
            if (prefetch && t0 + RC_TOK >= n && bh + 1 < last) {
                if constexpr (AHEAD) fetch(bh + 1);
                if (tok_ahead) fetch_tokens(bh + 1);
                fetched = true;
            }
            for (int tt = 0; tt < nt; ++tt) {
                const float4* k4 = reinterpret_cast<const float4*>(&sK[tt][rg * NE]);
                const float4* q4 = reinterpret_cast<const float4*>(&sQ[tt][rg * NE]);
                const float4* a4 = reinterpret_cast<const float4*>(&sA[tt][rg * NE]);
                float x = 0.f, y = 0.f;
#pragma unroll
                for (int i = 0; i < NE / 4; ++i) {
                    const float4 kk = k4[i], qq = q4[i], aa = a4[i];
                    s[4 * i] *= aa.x;
                    s[4 * i + 1] *= aa.y;
                    s[4 * i + 2] *= aa.z;
                    s[4 * i + 3] *= aa.w;
                    x = fmaf(kk.x, s[4 * i], x);
                    x = fmaf(kk.y, s[4 * i + 1], x);
                    x = fmaf(kk.z, s[4 * i + 2], x);
                    x = fmaf(kk.w, s[4 * i + 3], x);
                    y = fmaf(qq.x, s[4 * i], y);
                    y = fmaf(qq.y, s[4 * i + 1], y);
                    y = fmaf(qq.z, s[4 * i + 2], y);
                    y = fmaf(qq.w, s[4 * i + 3], y);
                }
                if constexpr (CPW == 8) {
                    x = add_xor32(add_xor16(add_xor8(x)));
                    y = add_xor32(add_xor16(add_xor8(y)));
                } else {
                    x = add_xor32(add_xor16(x));
                    y = add_xor32(add_xor16(y));
                }
                const float u = sB[tt] * (sV[tt][col] - x);
#pragma unroll
                for (int i = 0; i < NE / 4; ++i) {
                    const float4 kk = k4[i];
                    s[4 * i] = fmaf(kk.x, u, s[4 * i]);
                    s[4 * i + 1] = fmaf(kk.y, u, s[4 * i + 1]);
                    s[4 * i + 2] = fmaf(kk.z, u, s[4 * i + 2]);
                    s[4 * i + 3] = fmaf(kk.w, u, s[4 * i + 3]);
                }
                if (emit && rg == 0) {
                    const size_t row = ((size_t)b * src.T + t0 + tt) * H + h;
                    o[row * 128 + col] = fmaf(sQK[tt], u, y);
                }
            }
        }
    };

    for (; bh < last; ++bh) {
        b = bh / H;
        h = (int)(bh - b * H);
        // state -> LDS -> registers (the previous state's store has finished
        // reading the staging area)
        if constexpr (!AHEAD) fetch(bh);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NPF; ++j) {
            const int e = tid + RC_THREADS * j;
            *reinterpret_cast<f32x4*>(&sS[(e >> 5) * RC_LDS + 4 * (e & 31)]) = pf[j];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NE; ++i) s[i] = sS[(rg + RG * i) * RC_LDS + col];
        int nr = 0;
        if (rep.T > 0) {
            nr = n_replay ? n_replay[b] : rep.T;
            nr = nr < 0 ? 0 : (nr > rep.T ? rep.T : nr);
            run(rep, nr, false, false);
        }
        if (!commit && nr > 0) store_state();
        fetched = false;
        run(out, out.T, true, true);
        if constexpr (AHEAD)
            if (!fetched && bh + 1 < last) fetch(bh + 1);
        if (commit) store_state();
    }
}

hipError_t launch_recurrent(const void* q, const void* k, const void* v, bool bf16_in,
                            const float* log_alpha, const float* beta, const void* rq,
                            const void* rk, const void* rv, const float* rlog_alpha,
                            const float* rbeta, const int32_t* n_replay, float* S,
                            int64_t n_states, int32_t H, int32_t T, int32_t Tr, int32_t commit,
                            float* o, hipStream_t stream) {
    const TokSrc out{q, k, v, log_alpha, beta, T};
    const TokSrc rep{rq, rk, rv, rlog_alpha, rbeta, Tr};
    // several states per workgroup once there are enough to keep every
    // compute unit busy (at least eight workgroups each), so that state
    // reads overlap token work
    const int64_t fill = n_states / 2048;
    const int32_t per_wg = fill < 1 ? 1 : (fill > RC_MAX_PER_WG ? RC_MAX_PER_WG : (int32_t)fill);
    dim3 grid((unsigned)((n_states + per_wg - 1) / per_wg));
    const bool wide = (int64_t)T + Tr >= RC_WIDE_TOKENS;   // two workgroups per compute unit
#define KDA_RC(T_, C_)                                                                            \
    hipLaunchKernelGGL((recurrent_kernel<T_, C_>), grid, dim3(64 * 128 / C_), 0, stream, rep,     \
                       n_replay, out, S, o, H, commit, n_states, per_wg)
    if (bf16_in) {
        if (wide) KDA_RC(__bf16, 16);
        else KDA_RC(__bf16, 8);
    } else {
        if (wide) KDA_RC(float, 16);
        else KDA_RC(float, 8);
    }
#undef KDA_RC
    return hipGetLastError();
}

}  // namespace kda
