// Chunkwise KDA prefill (gfx950).
//
// Algebra: "尝试对Kimi KDA的数学推导&算子实现分析" (hjcheng0602.cn) eqs.
// (8)-(66), row-beta form.  Per chunk of C tokens with incoming state S:
//   g_t  = sum_{r<=t} log alpha_r (restarted at the chunk start)      (9)
//   L    = StrictTril(B_beta K+ K-^T),  k+ = k e^{g}, k- = k e^{-g}    (51)
//   U    = (I + L)^{-1} B_beta (V - K+ S)                              (52)
//   O    = Q+ S + Tril(Q+ K-^T) U                                      (63)
//   S   <- Diag(e^{g_C}) S + K_end^T U,  k_end = k e^{g_C - g}          (66)
//
// MI355X design (not the pages' two-kernel split):
//   * One workgroup (4 waves) per (sequence, head, value-column slice)
//     walks the sequence's chunks serially.  The recurrence acts on S from
//     the left, so value columns evolve independently: each wave owns
//     WCOLS columns of the 128 x 128 fp32 state and keeps them in MFMA
//     accumulator registers for the whole sequence; S never leaves the CU
//     until the final state is written.
//   * C = 32 tokens per chunk, split into two 16-token sub-tiles.  Every
//     e^{g_t - g_j} product is evaluated as (x e^{g_t - r}) (k e^{r - g_j})
//     with r the cumulative decay at a sub-tile boundary, so with
//     log alpha >= -5 ("Kimi K3 技术报告解读" section 3.5: a 16-token tile
//     stays within (-80, 0)) every factor lies in [e^-80, e^80]: no
//     overflow, and an underflowing factor multiplies one that is <= 1.
//   * Precision (bf16 inputs): products that can dominate an output use
//     split bf16 operands (hi + lo, 16 significant bits): the L / M tiles,
//     R, U, M and K_end.  K+, Q+, S and the diagonal blocks of T are
//     rounded once.  fp32 inputs use exact fp32 MFMA (16x16x4) throughout.
//   * Chunk-local tiles go through LDS twice-buffered so the next chunk's
//     decay scan never waits for the previous chunk's readers; two
//     workgroup barriers per chunk.  The next chunk's inputs are loaded
//     into registers while the current chunk computes.
//   * Grid: blockIdx -> (unit, slice) so that the slices of one head land
//     on the same XCD (blockIdx % 8) and share its L2; units are taken
//     longest sequence first when a sorted order is supplied.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int CH = 32;        // chunk length (tokens)
constexpr int DK = 128;       // key / value head dimension
constexpr int LDT = DK + 4;   // LDS row stride of token-major [CH][DK] tiles (floats)
constexpr int LDM = CH + 4;   // LDS row stride of [CH][CH] tiles (floats)
constexpr int PF_THREADS = 256;


template <typename InT>
struct PairOf;
template <>
struct PairOf<__bf16> {
    typedef uint32_t type;  // two packed bf16
};
template <>
struct PairOf<float> {
    typedef float2 type;
};

__device__ __forceinline__ float2 unpack2(uint32_t u) {
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}
__device__ __forceinline__ float2 unpack2(float2 f) { return f; }

template <typename InT, int WCOLS>
__global__ __launch_bounds__(PF_THREADS) void chunk_fwd_kernel(PrefillParams p) {
    constexpr bool F32 = std::is_same<InT, float>::value;
    constexpr int NCT = WCOLS / 16;   // 16-column tiles per wave
    constexpr int DVW = 4 * WCOLS;    // value columns per workgroup
    typedef typename PairOf<InT>::type Pair;

    // ---------------------------------------------------------------- work item
    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int slot = blk >> 3;
    const int slice = slot % p.n_slices;
    const int unit = (slot / p.n_slices) * 8 + xcd;
    if (unit >= p.n_units) return;
    const int rank = unit / p.H;
    const int h = unit - rank * p.H;
    const int n = p.order ? p.order[rank] : rank;
    const int64_t Tt = p.T;
    int64_t t0, t1;
    if (p.cu) {
        int64_t a = p.cu[n], b = p.cu[n + 1];
        t0 = a < 0 ? 0 : (a > Tt ? Tt : a);
        t1 = b < t0 ? t0 : (b > Tt ? Tt : b);
    } else {
        t0 = (int64_t)n * Tt;
        t1 = t0 + Tt;
    }
    const int H = p.H;
    const InT* __restrict__ qg = (const InT*)p.q;
    const InT* __restrict__ kg = (const InT*)p.k;
    const InT* __restrict__ vg = (const InT*)p.v;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;     // lane group
    const int ln = lane & 15;    // row / column within a 16-wide tile
    const int col0 = slice * DVW + wave * WCOLS;   // first value column of this wave

    __shared__ __attribute__((aligned(16))) float sKs[2][CH * LDT];  // k e^{g - r_start}
    __shared__ __attribute__((aligned(16))) float sQs[2][CH * LDT];  // q e^{g - r_start}
    __shared__ __attribute__((aligned(16))) float sKh[2][CH * LDT];  // k e^{r_end - g}
    // per channel: 0: e^{D0}, 1: e^{-D0}, 2: e^{D1}, 3: e^{-D1} where
    // D_b >= 0 is the decay magnitude accumulated over sub-tile b.
    __shared__ __attribute__((aligned(16))) float sVec[2][4][DK];
    __shared__ __attribute__((aligned(16))) float sL[CH * LDM];
    __shared__ __attribute__((aligned(16))) float sT[CH * LDM];
    __shared__ __attribute__((aligned(16))) float sM[CH * LDM];

    // M's upper-right 16 x 16 block is identically zero; never rewritten.
    sM[(tid >> 4) * LDM + 16 + (tid & 15)] = 0.f;

    // ------------------------------------------------------------ state in
    f32x4 S[8][NCT];
    const size_t sbase = ((size_t)n * H + h) * (DK * DK);
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[it][ct][r] = p.S0 ? p.S0[sbase + (size_t)(it * 16 + g * 4 + r) * DK + col0 +
                                           ct * 16 + ln]
                                    : 0.f;

    // -------------------------------------------------------- input loaders
    // Decay-scan role of this thread: wave>>1 selects k (0) or q (1),
    // wave&1 the sub-tile, lane the channel pair (2 lane, 2 lane + 1).
    const int kind = wave >> 1;
    const int sb = wave & 1;
    const InT* __restrict__ xg = kind ? qg : kg;
    Pair px[16];
    float2 pla[16];
    auto load_scan = [&](int64_t c0) {
#pragma unroll
        for (int tau = 0; tau < 16; ++tau) {
            const int64_t tok = c0 + sb * 16 + tau;
            if (tok < t1) {
                const size_t off = ((size_t)tok * H + h) * DK + 2 * lane;
                px[tau] = *reinterpret_cast<const Pair*>(xg + off);
                pla[tau] = *reinterpret_cast<const float2*>(p.la + off);
            } else {
                px[tau] = Pair{};
                pla[tau] = make_float2(0.f, 0.f);
            }
        }
    };
    // Values and beta in C layout for this wave's columns.
    InT pv[2][NCT][4];
    float pb[2][4];
    auto load_vb = [&](int64_t c0) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t tok = c0 + tb * 16 + g * 4 + r;
                const bool ok = tok < t1;
                pb[tb][r] = ok ? p.beta[(size_t)tok * H + h] : 0.f;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    pv[tb][ct][r] = ok ? vg[((size_t)tok * H + h) * DK + col0 + ct * 16 + ln]
                                       : (InT)0.f;
            }
    };

    load_scan(t0);
    load_vb(t0);

    int buf = 0;
    for (int64_t c0 = t0; c0 < t1; c0 += CH, buf ^= 1) {
        const int nvalid = (int)((t1 - c0) < CH ? (t1 - c0) : CH);
        float* Ks = sKs[buf];
        float* Qs = sQs[buf];
        float* Kh = sKh[buf];
        float(*Vec)[DK] = sVec[buf];

        // ------------------------------------------------ 1. decay scan
        // s_tau = sum of log alpha over the sub-tile up to token tau;
        // tile values x e^{s_tau} (<= 1) and, for k, k e^{s_15 - s_tau} (<= 1).
        {
            float cs0[16], cs1[16];
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int tau = 0; tau < 16; ++tau) {
                a0 += pla[tau].x;
                a1 += pla[tau].y;
                cs0[tau] = a0;
                cs1[tau] = a1;
            }
            float* dst = kind ? Qs : Ks;
#pragma unroll
            for (int tau = 0; tau < 16; ++tau) {
                const float2 x = unpack2(px[tau]);
                const int row = sb * 16 + tau;
                *reinterpret_cast<float2*>(dst + row * LDT + 2 * lane) =
                    make_float2(x.x * expf(cs0[tau]), x.y * expf(cs1[tau]));
                if (kind == 0)
                    *reinterpret_cast<float2*>(Kh + row * LDT + 2 * lane) =
                        make_float2(x.x * expf(a0 - cs0[tau]), x.y * expf(a1 - cs1[tau]));
            }
            if (kind == 0) {
                *reinterpret_cast<float2*>(&Vec[2 * sb][2 * lane]) = make_float2(expf(-a0), expf(-a1));
                *reinterpret_cast<float2*>(&Vec[2 * sb + 1][2 * lane]) = make_float2(expf(a0), expf(a1));
            }
        }
        if (c0 + CH < t1) load_scan(c0 + CH);   // next chunk's k/q/log alpha
        __syncthreads();

        // ------------------------------- 2. L and M tiles; K+ S and Q+ S
        // Block (b, a) of a C x C tile: left rows of sub-tile b (x e^{g - r_start(b)},
        // times e^{D_b} on the diagonal block so the reference is r_end(b) =
        // r_end(a)), right rows k e^{r_end(a) - g} of sub-tile a.
        auto block_mma = [&](const float* left, int lrow0, const float* scale, int rrow0) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int kk = ks * 32 + g * 8;
                float a[8], b[8];
                const float4* la4 = reinterpret_cast<const float4*>(left + (lrow0 + ln) * LDT + kk);
                const float4* rb4 = reinterpret_cast<const float4*>(Kh + (rrow0 + ln) * LDT + kk);
                float4 a0 = la4[0], a1 = la4[1], b0 = rb4[0], b1 = rb4[1];
                a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w;
                a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
                b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w;
                b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
                if (scale) {
                    const float4* s4 = reinterpret_cast<const float4*>(scale + kk);
                    float4 s0 = s4[0], s1 = s4[1];
                    a[0] *= s0.x; a[1] *= s0.y; a[2] *= s0.z; a[3] *= s0.w;
                    a[4] *= s1.x; a[5] *= s1.y; a[6] *= s1.z; a[7] *= s1.w;
                }
                mma_k32<F32, SPLIT2>(acc, a, b);
            }
            return acc;
        };

        if (wave == 0) {
            // L00, L11 -> invert the two unit-lower-triangular diagonal blocks.
            f32x4 l00 = block_mma(Ks, 0, Vec[0], 0);
            f32x4 l11 = block_mma(Ks, 16, Vec[2], 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = g * 4 + r;
                sL[row * LDM + ln] = ln < row ? pb[0][r] * l00[r] : 0.f;
                sL[(16 + row) * LDM + 16 + ln] = ln < row ? pb[1][r] * l11[r] : 0.f;
            }
            wave_lds_sync();
            if (lane < 32) {
                // Column j of (I + L_bb)^{-1} by forward substitution.
                const int bb = lane >> 4, j = lane & 15;
                const float* Lb = sL + (16 * bb) * LDM + 16 * bb;
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
                for (int c = 0; c < 15; ++c) {
                    const float xc = x[c];
#pragma unroll
                    for (int i = c + 1; i < 16; ++i) x[i] -= Lb[i * LDM + c] * xc;
                }
                float* Tb = sT + (16 * bb) * LDM + 16 * bb;
#pragma unroll
                for (int i = 0; i < 16; ++i) Tb[i * LDM + j] = x[i];
            }
        } else if (wave == 1) {
            f32x4 l10 = block_mma(Ks, 16, nullptr, 0);
            f32x4 m00 = block_mma(Qs, 0, Vec[0], 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = g * 4 + r;
                sL[(16 + row) * LDM + ln] = pb[1][r] * l10[r];
                sM[row * LDM + ln] = ln <= row ? m00[r] : 0.f;
            }
        } else if (wave == 2) {
            f32x4 m10 = block_mma(Qs, 16, nullptr, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) sM[(16 + g * 4 + r) * LDM + ln] = m10[r];
        } else {
            f32x4 m11 = block_mma(Qs, 16, Vec[2], 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = g * 4 + r;
                sM[(16 + row) * LDM + 16 + ln] = ln <= row ? m11[r] : 0.f;
            }
        }

        // K+ S -> R and Q+ S -> O for this wave's columns (state at chunk start).
        // k+ of sub-tile 1 = (k e^{g - r_end(0)}) e^{-D0}.
        f32x4 R[2][NCT], O[2][NCT];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                R[tb][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                O[tb][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            Frag8 bS[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    bS[ct].f[r] = S[2 * ks][ct][r];
                    bS[ct].f[4 + r] = S[2 * ks + 1][ct][r];
                }
                prep8<F32, PLAIN>(bS[ct]);
            }
            const int k0 = ks * 32 + g * 4;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                Frag8 aK, aQ;
                const float* kr = Ks + (tb * 16 + ln) * LDT;
                const float* qr = Qs + (tb * 16 + ln) * LDT;
                float4 k0v = *reinterpret_cast<const float4*>(kr + k0);
                float4 k1v = *reinterpret_cast<const float4*>(kr + k0 + 16);
                float4 q0v = *reinterpret_cast<const float4*>(qr + k0);
                float4 q1v = *reinterpret_cast<const float4*>(qr + k0 + 16);
                float4 s0v = make_float4(1.f, 1.f, 1.f, 1.f), s1v = s0v;
                if (tb == 1) {
                    s0v = *reinterpret_cast<const float4*>(&Vec[1][k0]);
                    s1v = *reinterpret_cast<const float4*>(&Vec[1][k0 + 16]);
                }
                aK.f[0] = k0v.x * s0v.x; aK.f[1] = k0v.y * s0v.y; aK.f[2] = k0v.z * s0v.z; aK.f[3] = k0v.w * s0v.w;
                aK.f[4] = k1v.x * s1v.x; aK.f[5] = k1v.y * s1v.y; aK.f[6] = k1v.z * s1v.z; aK.f[7] = k1v.w * s1v.w;
                aQ.f[0] = q0v.x * s0v.x; aQ.f[1] = q0v.y * s0v.y; aQ.f[2] = q0v.z * s0v.z; aQ.f[3] = q0v.w * s0v.w;
                aQ.f[4] = q1v.x * s1v.x; aQ.f[5] = q1v.y * s1v.y; aQ.f[6] = q1v.z * s1v.z; aQ.f[7] = q1v.w * s1v.w;
                prep8<F32, PLAIN>(aK);
                prep8<F32, PLAIN>(aQ);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    mma_k32<F32, PLAIN>(R[tb][ct], aK, bS[ct]);
                    mma_k32<F32, PLAIN>(O[tb][ct], aQ, bS[ct]);
                }
            }
        }
        __syncthreads();

        // --------------------------------------- 3. U, O and the state update
        // R' = B_beta (V - K+ S)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    R[tb][ct][r] = pb[tb][r] * (to_f32(pv[tb][ct][r]) - R[tb][ct][r]);

        // Block forward substitution with the diagonal inverses:
        // U0 = T00 R'0 ; U1 = T11 (R'1 - L10 U0).
        f32x4 U0[NCT], U1[NCT];
        {
            float t00[4], nl10[4], t11[4];
            float4 a = *reinterpret_cast<const float4*>(sT + ln * LDM + g * 4);
            t00[0] = a.x; t00[1] = a.y; t00[2] = a.z; t00[3] = a.w;
            a = *reinterpret_cast<const float4*>(sL + (16 + ln) * LDM + g * 4);
            nl10[0] = -a.x; nl10[1] = -a.y; nl10[2] = -a.z; nl10[3] = -a.w;
            a = *reinterpret_cast<const float4*>(sT + (16 + ln) * LDM + 16 + g * 4);
            t11[0] = a.x; t11[1] = a.y; t11[2] = a.z; t11[3] = a.w;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                float b[4];
                U0[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 4; ++r) b[r] = R[0][ct][r];
                mma_k16<F32, SPLITB>(U0[ct], t00, b);
                f32x4 X = R[1][ct];
#pragma unroll
                for (int r = 0; r < 4; ++r) b[r] = U0[ct][r];
                mma_k16<F32, SPLITB>(X, nl10, b);
                U1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < 4; ++r) b[r] = X[r];
                mma_k16<F32, SPLITB>(U1[ct], t11, b);
            }
        }

        // U as the B operand of M U and K_end^T U (tile order: U0 rows then U1 rows).
        Frag8 bU[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bU[ct].f[r] = U0[ct][r];
                bU[ct].f[4 + r] = U1[ct][r];
            }
            prep8<F32, SPLIT2>(bU[ct]);
        }

        // O = Q+ S + M U, written for the valid rows.
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            Frag8 aM;
            const float* mr = sM + (tb * 16 + ln) * LDM + g * 4;
            float4 m0 = *reinterpret_cast<const float4*>(mr);
            float4 m1 = *reinterpret_cast<const float4*>(mr + 16);
            aM.f[0] = m0.x; aM.f[1] = m0.y; aM.f[2] = m0.z; aM.f[3] = m0.w;
            aM.f[4] = m1.x; aM.f[5] = m1.y; aM.f[6] = m1.z; aM.f[7] = m1.w;
            prep8<F32, SPLIT2>(aM);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                mma_k32<F32, SPLIT2>(O[tb][ct], aM, bU[ct]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = tb * 16 + g * 4 + r;
                    if (row < nvalid)
                        p.o[((size_t)(c0 + row) * H + h) * DK + col0 + ct * 16 + ln] = O[tb][ct][r];
                }
            }
        }

        // S <- Diag(e^{g_C}) S + K_end^T U with e^{g_C} = e^{-D0} e^{-D1} and
        // k_end = (k e^{r_end(b) - g}) times e^{-D1} for sub-tile 0.
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int i = it * 16 + ln;
            const float e1 = Vec[3][i];
            Frag8 aKe;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                aKe.f[e] = Kh[(g * 4 + e) * LDT + i] * e1;
                aKe.f[4 + e] = Kh[(16 + g * 4 + e) * LDT + i];
            }
            prep8<F32, SPLIT2>(aKe);
            float dec[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = it * 16 + g * 4 + r;
                dec[r] = Vec[1][row] * Vec[3][row];
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[it][ct][r] *= dec[r];
                mma_k32<F32, SPLIT2>(S[it][ct], aKe, bU[ct]);
            }
        }

        if (c0 + CH < t1) load_vb(c0 + CH);   // next chunk's v / beta
    }

    // ------------------------------------------------------------ state out
    if (p.S_T) {
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.S_T[sbase + (size_t)(it * 16 + g * 4 + r) * DK + col0 + ct * 16 + ln] =
                        S[it][ct][r];
    }
}

// Longest-first order of the packed sequences: order[rank] = sequence, with
// rank = number of sequences that are longer, or as long with a smaller
// index.  O(n^2) comparisons, used only for n <= kOrderMax.
__global__ void seq_order_kernel(const int32_t* __restrict__ cu, int32_t n, int64_t T,
                                 int32_t* __restrict__ order) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    auto len = [&](int s) -> int64_t {
        int64_t a = cu[s], b = cu[s + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
        return b - a;
    };
    const int64_t li = len(i);
    int rank = 0;
    for (int j = 0; j < n; ++j) {
        const int64_t lj = len(j);
        rank += (lj > li) || (lj == li && j < i);
    }
    order[rank] = i;
}

hipError_t launch_chunk_fwd(const PrefillParams& prm, bool bf16_in, int wcols, bool sort,
                            hipStream_t stream) {
    PrefillParams p = prm;
    if (sort && p.cu) {
        const int thr = 256;
        hipLaunchKernelGGL(seq_order_kernel, dim3((p.n_seqs + thr - 1) / thr), dim3(thr), 0,
                           stream, p.cu, p.n_seqs, p.T, const_cast<int32_t*>(p.order));
    } else {
        p.order = nullptr;
    }
    const int64_t groups = ((int64_t)p.n_units + 7) / 8;
    dim3 grid((unsigned)(groups * 8 * p.n_slices)), block(PF_THREADS);
    if (bf16_in) {
        if (wcols == 32)
            hipLaunchKernelGGL((chunk_fwd_kernel<__bf16, 32>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((chunk_fwd_kernel<__bf16, 16>), grid, block, 0, stream, p);
    } else {
        if (wcols == 32)
            hipLaunchKernelGGL((chunk_fwd_kernel<float, 32>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((chunk_fwd_kernel<float, 16>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace kda
