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
// This kernel runs fp32 inputs, and bf16 inputs with 32 value columns per
// consumer wave (one workgroup per head: with 256 or more (sequence, head)
// units, and for the sequence-parallel path's dual-chain pass and the rerun
// of its middle segments); bf16 with two 64-column slices per head runs the
// pipelined kernel of kda_prefill_pipe.hip instead.
//
// MI355X design (not the pages' two-kernel split):
//   * One workgroup (4 consumer waves and NPROD producer waves) per
//     (sequence, head, value-column slice) walks the sequence's chunks
//     serially.  The recurrence acts on S from the left, so value columns
//     evolve independently: each consumer wave owns WCOLS columns of the
//     128 x 128 fp32 state and keeps them in MFMA accumulator registers for
//     the whole sequence.
//   * C = 32 tokens per chunk.  Every decay product is factored about the
//     cumulative decay E0 at the end of the chunk's first 16 tokens:
//         X = k e^{g - E0},  QX = q e^{g - E0},  Y = k e^{E0 - g},
//     so k+_t . k-_j = X_t . Y_j for all j <= t in the chunk.  With
//     log alpha >= -5 ("Kimi K3 技术报告解读" section 3.5: 16 tokens stay
//     within (-80, 0)) every factor lies in [e^-80, e^80] and each product
//     with j <= t is <= 1: no overflow, and an underflowing factor only
//     ever multiplies one that is <= 1.  The chunk-level operands follow
//     by per-channel scalings of the state instead of more tiles:
//         K+ S = X (e^{E0} S),  Q+ S = QX (e^{E0} S),
//         S_next = e^{E1 - E0} (e^{E0} S + Y^T U)   (E1 = g_C).
//   * The decay scan and the operand tiles are produced once per chunk by
//     the producer waves (two key channels and 32 / NPROD tokens per lane;
//     the parts of a 16-token sub-tile exchange partial sums across the wave) directly
//     in the MFMA operand layouts (token-major rows for the products over
//     channels, channel-major rows of Y for the product over tokens), so
//     the matrix loops only load and issue.  Inputs arrive through buffer
//     loads whose range ends at the sequence's last token (out-of-range
//     rows read as zero, no branches).
//   * bf16 inputs: X (for L and K+ S), QX (for Q+ S) and T are rounded
//     once; QX and Y are split into hi + lo bf16 pairs for
//     M = Tril(QX Y^T) (whose near-diagonal entries dominate o), and the
//     state (in K+ S, Q+ S), V - K+S, U, M and Y^T (state update) are split
//     as well.  fp32 inputs
//     use fp32 MFMA (16x16x4) everywhere with fp32 tiles.
//   * Two workgroup barriers per chunk.  The state-dependent chain of
//     chunk c and the decay scan of chunk c+1 share a barrier interval, so
//     each wave interleaves matrix-core and vector work.  Inputs are
//     prefetched into registers one chunk ahead.
//   * Grid: blockIdx -> (unit, slice) so that the slices of one head land
//     on the same XCD (blockIdx % 8) and share its L2; units are taken
//     longest sequence first when a sorted order is supplied.
#include "kda_chunk.h"
#include "kda_launch.h"

namespace kda {

// NPROD producer waves (4 or 8) follow the 4 consumer waves.  DUAL: every
// consumer wave carries two chains over the same tiles, the one from S0 (or
// zero) with the values v (final state -> S_T) and the one from the identity
// with v read as zero (final state = the transition -> S_T2); o is not
// formed.
template <typename InT, int WCOLS, int NPROD, bool STORE_H, bool DUAL = false>
__global__ __launch_bounds__(64 * (4 + NPROD)) void chunk_fwd_kernel(PrefillParams p) {
    constexpr bool F32 = std::is_same<InT, float>::value;
    static_assert(!(DUAL && STORE_H), "the dual chain keeps no per-chunk states");
    constexpr int NCT = WCOLS / 16;   // 16-column tiles per consumer wave
    constexpr int DVW = 4 * WCOLS;    // value columns per workgroup
    constexpr int ES = (int)sizeof(InT);
    typedef Tiles<F32> TL;
    typedef typename TL::Op Op;
    constexpr int LDR = TL::LDR, LDY = TL::LDY;

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
        const int64_t b = p.seg_sel >= 0 ? n : n / p.seg_per_seq;
        const int64_t r = p.seg_sel >= 0 ? p.seg_sel : p.seg_r0 + (n - b * p.seg_per_seq);
        const int64_t first = p.seg_first > 0 ? p.seg_first : p.seg_len;
        const int64_t len = r == 0 ? first : p.seg_len;
        const int64_t e = (b + 1) * Tt;
        t0 = b * Tt + (r == 0 ? 0 : first + (r - 1) * p.seg_len);
        t0 = t0 < e ? t0 : e;
        t1 = e - t0 > len ? t0 + len : e;
    }
    const int64_t nch = (t1 - t0 + CH - 1) / CH;
    // STORE_H outputs: first state slot of this chain and the offset added to
    // its token rows (window mode: the compact layout described at seg_sel)
    const int64_t hslot0 = p.seg_sel >= 0 ? (int64_t)n * (p.seg_len / CH) : t0 / CH + n;
    const int64_t srow = p.seg_sel >= 0 ? (int64_t)n * p.seg_len - t0 : 0;
    const int H = p.H;
    const int rowel = H * DK;   // elements between consecutive tokens

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const bool consumer = wave < 4;
    const int role = consumer ? wave : wave - 4;   // consumer column block / producer role
    const int g = lane >> 4;     // lane group
    const int ln = lane & 15;    // row / column within a 16-wide tile
    const int col0 = slice * DVW + role * WCOLS;   // first value column (consumers)

    // ------------------------------------------------------------------ LDS
    // Buffers indexed [chunk & 1] are written by the producers one step
    // before the consumers read them; the others live within one step.
    __shared__ __attribute__((aligned(16))) Op sX[2][CH * LDR];    // k e^{g - E0}
    __shared__ __attribute__((aligned(16))) Op sQX[2][CH * LDR];   // q e^{g - E0} (hi)
    __shared__ __attribute__((aligned(16))) Op sY[CH * LDR];       // k e^{E0 - g} (hi)
    __shared__ __attribute__((aligned(16))) Op sQXl[F32 ? 4 : CH * LDR];   // lo parts
    __shared__ __attribute__((aligned(16))) Op sYl[F32 ? 4 : CH * LDR];
    __shared__ __attribute__((aligned(16))) Op sYt[2][DK * LDY];               // Y^T hi
    __shared__ __attribute__((aligned(16))) Op sYtl[2][F32 ? 4 : DK * LDY];    // Y^T lo
    __shared__ __attribute__((aligned(16))) float sVec[2][2][DK];  // e^{E0}, e^{E1 - E0}
    __shared__ __attribute__((aligned(16))) float sL[CH * LDM];    // beta-scaled L blocks 00, 11
    __shared__ __attribute__((aligned(16))) float sT[2][CH * LDM]; // T00, T11 and -L10 (beta-scaled)
    // M = Tril(Q+ K-^T): bf16 path as packed (hi | lo << 16) pairs, fp32 path as floats.
    __shared__ __attribute__((aligned(16))) uint32_t sM[2][CH * LDM];

    // M's upper-right 16 x 16 block is identically zero; never rewritten.
    if (tid < 512) sM[tid >> 8][((tid & 255) >> 4) * LDM + 16 + (tid & 15)] = 0u;

    auto n_valid = [&](int64_t c) -> int {
        const int64_t nv = t1 - c;
        return nv <= 0 ? 0 : (nv < CH ? (int)nv : CH);
    };
    auto span_bytes = [&](int nv, int es) -> int {
        return nv <= 0 ? 0 : ((nv - 1) * rowel + DK) * es;
    };
    // beta of a chunk in C layout (rows tb*16 + 4g + r), 0 past the end.
    auto load_beta = [&](int64_t cidx, float (&b)[2][4]) {
        const int64_t c = t0 + cidx * CH;
        const int nv = n_valid(c);
        const auto rb = make_rsrc(p.beta + (size_t)c * H + h, nv <= 0 ? 0 : ((nv - 1) * H + 1) * 4);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                b[tb][r] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rb, (tb * 16 + g * 4 + r) * H * 4, 0, 0));
    };

    // ======================================================== consumer state
    f32x4 S[8][NCT];
    f32x4 S2[DUAL ? 8 : 1][DUAL ? NCT : 1];   // the identity-start chain
    const size_t sbase = ((size_t)n * H + h) * (DK * DK);
    float pv[2][NCT][4], pb[2][4];
    auto load_v = [&](int64_t cidx, float (&v)[2][NCT][4]) {
        const int64_t c = t0 + cidx * CH;
        const int nv = n_valid(c);
        const auto rv = make_rsrc((const InT*)p.v + ((size_t)c * H + h) * DK,
                                  p.s0_identity ? 0 : span_bytes(nv, ES));
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const int el = (tb * 16 + g * 4 + r) * rowel + col0 + ct * 16 + ln;
                    if constexpr (F32)
                        v[tb][ct][r] = __uint_as_float(
                            __builtin_amdgcn_raw_buffer_load_b32(rv, el * 4, 0, 0));
                    else
                        v[tb][ct][r] = __uint_as_float(
                            (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rv, el * 2, 0, 0) << 16);
                }
    };
    // Chain values carried from phase A to phase B of a step.
    f32x4 O[2][NCT], U0[NCT], U1[NCT];
    Frag<F32> bUh[NCT], bUl[NCT];
    Frag<F32> bUh2[DUAL ? NCT : 1], bUl2[DUAL ? NCT : 1];

    // ======================================================== producer state
    // Scan role: a lane handles TPL consecutive tokens of the channel pair
    // (2 cp, 2 cp + 1); the PARTS lanes holding one pair (lane stride LPP)
    // cover the 16-token sub-tile sb.
    constexpr int TPL = 32 / NPROD;     // tokens per lane
    constexpr int PARTS = 16 / TPL;     // lanes per channel pair and sub-tile
    constexpr int LPP = 64 / PARTS;     // channel pairs per wave
    constexpr int WPS = NPROD / 2;      // waves per sub-tile
    const int sb = role / WPS;
    const int cp = (role % WPS) * LPP + lane % LPP;
    const int part = lane / LPP;
    const int sc = 2 * cp;
    typedef typename std::conditional<F32, float2, uint32_t>::type Pair;
    Pair xk[TPL], xq[TPL];
    float2 xl[TPL];
    float pbp[2][4];   // beta of the chunk being prepared (loaded one step ahead)
    // Loads of one chunk's k, q (channel pair) and log alpha, one token at a
    // time, so that the scan can refill each register right after its last
    // use and the next chunk's loads overlap this chunk's arithmetic.
    struct ScanSrc {
        __amdgpu_buffer_rsrc_t k, q, l;
    };
    auto scan_src = [&](int64_t cidx) {
        const int64_t c = t0 + cidx * CH;
        const int nv = n_valid(c);
        const size_t eoff = ((size_t)c * H + h) * DK;
        return ScanSrc{make_rsrc((const InT*)p.k + eoff, span_bytes(nv, ES)),
                       make_rsrc((const InT*)p.q + eoff, span_bytes(nv, ES)),
                       make_rsrc(p.la + eoff, span_bytes(nv, 4))};
    };
    auto load_kq = [&](const ScanSrc& r, int tau) {
        const int el = (sb * 16 + part * TPL + tau) * rowel + sc;
        if constexpr (F32) {
            auto a = __builtin_amdgcn_raw_buffer_load_b64(r.k, el * 4, 0, 0);
            auto b = __builtin_amdgcn_raw_buffer_load_b64(r.q, el * 4, 0, 0);
            xk[tau] = make_float2(__uint_as_float(a[0]), __uint_as_float(a[1]));
            xq[tau] = make_float2(__uint_as_float(b[0]), __uint_as_float(b[1]));
        } else {
            xk[tau] = __builtin_amdgcn_raw_buffer_load_b32(r.k, el * 2, 0, 0);
            xq[tau] = __builtin_amdgcn_raw_buffer_load_b32(r.q, el * 2, 0, 0);
        }
    };
    auto load_la = [&](const ScanSrc& r, int tau) {
        const int el = (sb * 16 + part * TPL + tau) * rowel + sc;
        auto lv = __builtin_amdgcn_raw_buffer_load_b64(r.l, el * 4, 0, 0);
        xl[tau] = make_float2(__uint_as_float(lv[0]), __uint_as_float(lv[1]));
    };
    auto load_scan = [&](int64_t cidx) {
        const ScanSrc r = scan_src(cidx);
#pragma unroll
        for (int tau = 0; tau < TPL; ++tau) {
            load_kq(r, tau);
            load_la(r, tau);
        }
    };

    // Decay scan: writes X, QX (buffer `buf`), Y and the lo parts (single),
    // Y^T (buffer `buf`) and the per-channel scalings of buffer `buf`.
    auto scan = [&](int buf, int64_t cnext) {
        const ScanSrc nx = scan_src(cnext);
        float cs0[TPL], cs1[TPL];
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int tau = 0; tau < TPL; ++tau) {
            a0 += xl[tau].x * LOG2E;
            a1 += xl[tau].y * LOG2E;
            cs0[tau] = a0;
            cs1[tau] = a1;
        }
#pragma unroll
        for (int tau = 0; tau < TPL; ++tau) load_la(nx, tau);
        float pre0, pre1, tot0, tot1;
        parts_scan<PARTS>(a0, part, pre0, tot0);
        parts_scan<PARTS>(a1, part, pre1, tot1);
        const float ref0 = sb == 0 ? tot0 : 0.f, ref1 = sb == 0 ? tot1 : 0.f;
        if (part == 0)
            *reinterpret_cast<float2*>(&sVec[buf][sb][sc]) =
                make_float2(__builtin_amdgcn_exp2f(tot0), __builtin_amdgcn_exp2f(tot1));
        const int tc = sb * 16 + part * TPL;
        Op* X = sX[buf];
        Op* QX = sQX[buf];
        if constexpr (F32) {
            float y0[TPL], y1[TPL];
#pragma unroll
            for (int tau = 0; tau < TPL; ++tau) {
                const float d0 = cs0[tau] + pre0 - ref0, d1 = cs1[tau] + pre1 - ref1;
                const float fx0 = __builtin_amdgcn_exp2f(d0), fx1 = __builtin_amdgcn_exp2f(d1);
                const float fy0 = __builtin_amdgcn_exp2f(-d0), fy1 = __builtin_amdgcn_exp2f(-d1);
                const float2 kf = xk[tau], qf = xq[tau];
                load_kq(nx, tau);
                const int row = tc + tau;
                *reinterpret_cast<float2*>(&X[row * LDR + sc]) = make_float2(kf.x * fx0, kf.y * fx1);
                *reinterpret_cast<float2*>(&QX[row * LDR + sc]) = make_float2(qf.x * fx0, qf.y * fx1);
                y0[tau] = kf.x * fy0;
                y1[tau] = kf.y * fy1;
                *reinterpret_cast<float2*>(&sY[row * LDR + sc]) = make_float2(y0[tau], y1[tau]);
            }
#pragma unroll
            for (int i = 0; i < TPL / 4; ++i) {
                *reinterpret_cast<float4*>(&sYt[buf][sc * LDY + tc + 4 * i]) =
                    make_float4(y0[4 * i], y0[4 * i + 1], y0[4 * i + 2], y0[4 * i + 3]);
                *reinterpret_cast<float4*>(&sYt[buf][(sc + 1) * LDY + tc + 4 * i]) =
                    make_float4(y1[4 * i], y1[4 * i + 1], y1[4 * i + 2], y1[4 * i + 3]);
            }
        } else {
            uint32_t yh[TPL], yl[TPL];
#pragma unroll
            for (int tau = 0; tau < TPL; ++tau) {
                const float d0 = cs0[tau] + pre0 - ref0, d1 = cs1[tau] + pre1 - ref1;
                const float fx0 = __builtin_amdgcn_exp2f(d0), fx1 = __builtin_amdgcn_exp2f(d1);
                const float fy0 = __builtin_amdgcn_exp2f(-d0), fy1 = __builtin_amdgcn_exp2f(-d1);
                const float2 kf = bf2_to_f2(xk[tau]), qf = bf2_to_f2(xq[tau]);
                load_kq(nx, tau);
                const float X0 = kf.x * fx0, X1 = kf.y * fx1;
                const float Q0 = qf.x * fx0, Q1 = qf.y * fx1;
                const float Y0 = kf.x * fy0, Y1 = kf.y * fy1;
                const uint32_t qh = f2_to_bf2(Q0, Q1);
                yh[tau] = f2_to_bf2(Y0, Y1);
                const float2 qhf = bf2_to_f2(qh), yhf = bf2_to_f2(yh[tau]);
                yl[tau] = f2_to_bf2(Y0 - yhf.x, Y1 - yhf.y);
                const int row = tc + tau;
                *reinterpret_cast<uint32_t*>(&X[row * LDR + sc]) = f2_to_bf2(X0, X1);
                *reinterpret_cast<uint32_t*>(&QX[row * LDR + sc]) = qh;
                *reinterpret_cast<uint32_t*>(&sQXl[row * LDR + sc]) = f2_to_bf2(Q0 - qhf.x, Q1 - qhf.y);
                *reinterpret_cast<uint32_t*>(&sY[row * LDR + sc]) = yh[tau];
                *reinterpret_cast<uint32_t*>(&sYl[row * LDR + sc]) = yl[tau];
            }
            // Y^T rows sc and sc + 1: regroup the channel pairs into runs of
            // TPL tokens per channel.
            uint32_t h0[TPL / 2], h1[TPL / 2], l0[TPL / 2], l1[TPL / 2];
#pragma unroll
            for (int i = 0; i < TPL / 2; ++i) {
                h0[i] = perm2(yh[2 * i + 1], yh[2 * i], LO_HALVES);
                h1[i] = perm2(yh[2 * i + 1], yh[2 * i], HI_HALVES);
                l0[i] = perm2(yl[2 * i + 1], yl[2 * i], LO_HALVES);
                l1[i] = perm2(yl[2 * i + 1], yl[2 * i], HI_HALVES);
            }
            if constexpr (TPL == 8) {
                *reinterpret_cast<uint4*>(&sYt[buf][sc * LDY + tc]) = make_uint4(h0[0], h0[1], h0[2], h0[3]);
                *reinterpret_cast<uint4*>(&sYt[buf][(sc + 1) * LDY + tc]) = make_uint4(h1[0], h1[1], h1[2], h1[3]);
                *reinterpret_cast<uint4*>(&sYtl[buf][sc * LDY + tc]) = make_uint4(l0[0], l0[1], l0[2], l0[3]);
                *reinterpret_cast<uint4*>(&sYtl[buf][(sc + 1) * LDY + tc]) = make_uint4(l1[0], l1[1], l1[2], l1[3]);
            } else {
                *reinterpret_cast<uint2*>(&sYt[buf][sc * LDY + tc]) = make_uint2(h0[0], h0[1]);
                *reinterpret_cast<uint2*>(&sYt[buf][(sc + 1) * LDY + tc]) = make_uint2(h1[0], h1[1]);
                *reinterpret_cast<uint2*>(&sYtl[buf][sc * LDY + tc]) = make_uint2(l0[0], l0[1]);
                *reinterpret_cast<uint2*>(&sYtl[buf][(sc + 1) * LDY + tc]) = make_uint2(l1[0], l1[1]);
            }
        }
    };

    // 16 x 16 block of A B^T over the 128 channels (contiguous k order);
    // with `split`: A B^T = Ah Bh^T + Ah Bl^T + Al Bh^T.
    auto block = [&](const Op* A, const Op* Al, int arow0, const Op* B, const Op* Bl, int brow0,
                     bool split) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ao = (arow0 + ln) * LDR + ks * 32 + g * 8;
            const int bo = (brow0 + ln) * LDR + ks * 32 + g * 8;
            Frag<F32> a, b;
            load_contig(a, A + ao);
            load_contig(b, B + bo);
            if constexpr (!F32) {
                if (split) {
                    Frag<F32> al, bl;
                    load_contig(al, Al + ao);
                    load_contig(bl, Bl + bo);
                    mma(acc, al, b);
                    mma(acc, a, bl);
                }
            }
            mma(acc, a, b);
        }
        return acc;
    };
    // Store an M block (C layout) at rows r0, columns c0, keeping j <= t if diag.
    auto store_m = [&](uint32_t* Mb, const f32x4& m, int r0, int c0, bool diag) {
        uint32_t w[4];
        if constexpr (F32) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                w[r] = __float_as_uint((!diag || ln <= g * 4 + r) ? m[r] : 0.f);
        } else {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (!diag || ln <= g * 4 + r) ? m[r] : 0.f;
            const uint32_t h01 = f2_to_bf2(v[0], v[1]), h23 = f2_to_bf2(v[2], v[3]);
            const float2 f01 = bf2_to_f2(h01), f23 = bf2_to_f2(h23);
            const uint32_t l01 = f2_to_bf2(v[0] - f01.x, v[1] - f01.y);
            const uint32_t l23 = f2_to_bf2(v[2] - f23.x, v[3] - f23.y);
            w[0] = perm2(l01, h01, LO_HALVES);
            w[1] = perm2(l01, h01, HI_HALVES);
            w[2] = perm2(l23, h23, LO_HALVES);
            w[3] = perm2(l23, h23, HI_HALVES);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Mb[(r0 + g * 4 + r) * LDM + c0 + ln] = w[r];
    };

    // ------------------------------------------------------------ main loop
    // Step s: producers prepare chunk s while consumers finish chunk s - 1.
    // Each role runs its own loop over nch + 1 steps with two workgroup
    // barriers per step; the role is wave-uniform, so the barrier counts match.
    if (consumer) {
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[it][ct][r] = p.s0_identity
                                       ? (it * 16 + g * 4 + r == col0 + ct * 16 + ln ? 1.f : 0.f)
                                   : p.S0 ? p.S0[sbase + (size_t)(it * 16 + g * 4 + r) * DK + col0 +
                                                 ct * 16 + ln]
                                          : 0.f;
        if constexpr (DUAL) {
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        S2[it][ct][r] = it * 16 + g * 4 + r == col0 + ct * 16 + ln ? 1.f : 0.f;
        }
        // state at the start of chunk j -> slot hslot0 + j
        float* hbase = nullptr;
        if constexpr (STORE_H) hbase = p.h_states + ((size_t)hslot0 * H + h) * (DK * DK);
        auto store_h = [&](float* dst, int it, int ct) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[(size_t)(it * 16 + g * 4 + r) * DK + col0 + ct * 16 + ln] = S[it][ct][r];
        };
        if constexpr (STORE_H) {
            if (nch > 0) {
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) store_h(hbase, it, ct);
            }
        }
        load_v(0, pv);
        load_beta(0, pb);
        __syncthreads();   // step 0: nothing to finish yet
        __syncthreads();
        for (int64_t cidx = 0; cidx < nch; ++cidx) {
            // ---------------------------------------------------- phase A
            const int buf = (int)(cidx & 1);
            // S~ = e^{E0} S (for later chunks the previous update applied it)
            if (cidx == 0) {
                const float* e0 = sVec[buf][0];
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    const float4 sc4 = *reinterpret_cast<const float4*>(e0 + it * 16 + g * 4);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        S[it][ct][0] *= sc4.x;
                        S[it][ct][1] *= sc4.y;
                        S[it][ct][2] *= sc4.z;
                        S[it][ct][3] *= sc4.w;
                        if constexpr (DUAL) {
                            S2[it][ct][0] *= sc4.x;
                            S2[it][ct][1] *= sc4.y;
                            S2[it][ct][2] *= sc4.z;
                            S2[it][ct][3] *= sc4.w;
                        }
                    }
                }
            }
            // K+ S -> R and Q+ S -> O (DUAL: K+ S of both chains, no O)
            f32x4 R[2][NCT], R2[2][DUAL ? NCT : 1];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    R[tb][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                    O[tb][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if constexpr (DUAL) R2[tb][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            // the k-slice ks of a chain's state as the B operand (hi, lo)
            auto state_op = [&](const f32x4 (&St)[8][NCT], int ks, int ct, Frag<F32>& hi,
                                Frag<F32>& lo) {
                float f[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    f[r] = St[2 * ks][ct][r];
                    f[4 + r] = St[2 * ks + 1][ct][r];
                }
                if constexpr (F32) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) hi.v[e] = f[e];
                } else {
                    SplitBF<8> s8 = split8(f);
                    hi.v = s8.hi;
                    lo.v = s8.lo;
                }
            };
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                Frag<F32> bS[NCT], bSl[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) state_op(S, ks, ct, bS[ct], bSl[ct]);
                if constexpr (DUAL) {
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) {
                        Frag<F32> aK;
                        load_tile(aK, sX[buf] + (tb * 16 + ln) * LDR + ks * 32 + g * 4);
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            if constexpr (!F32) mma(R[tb][ct], aK, bSl[ct]);
                            mma(R[tb][ct], aK, bS[ct]);
                        }
                    }
                } else {
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) {
                        Frag<F32> aK, aQ;
                        load_tile(aK, sX[buf] + (tb * 16 + ln) * LDR + ks * 32 + g * 4);
                        load_tile(aQ, sQX[buf] + (tb * 16 + ln) * LDR + ks * 32 + g * 4);
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            if constexpr (!F32) {
                                mma(R[tb][ct], aK, bSl[ct]);
                                mma(O[tb][ct], aQ, bSl[ct]);
                            }
                            mma(R[tb][ct], aK, bS[ct]);
                            mma(O[tb][ct], aQ, bS[ct]);
                        }
                    }
                }
            }
            // R' = B_beta (V - K+ S)  (V - K+ S itself kept for the backward pass)
            if constexpr (STORE_H) {
                const int64_t cs = t0 + cidx * CH;
                const auto rr = make_rsrc(p.r_out + ((size_t)(cs + srow) * H + h) * DK, span_bytes(n_valid(cs), 4));
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int el = (tb * 16 + g * 4 + r) * rowel + col0 + ct * 16 + ln;
                            __builtin_amdgcn_raw_buffer_store_b32(
                                __float_as_uint(pv[tb][ct][r] - R[tb][ct][r]), rr, el * 4, 0, 0);
                        }
            }
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) R[tb][ct][r] = pb[tb][r] * (pv[tb][ct][r] - R[tb][ct][r]);
            // next chunk's values and beta (used one step later)
            load_v(cidx + 1, pv);
            load_beta(cidx + 1, pb);
            // Block forward substitution of (I + L) U = R':
            //   U0 = T00 R'0,  U1 = T11 (R'1 - L10 U0)
            {
                const float* Tb = sT[buf];
                float t00[4], t11[4], nl10[4];
                float4 a = *reinterpret_cast<const float4*>(Tb + ln * LDM + g * 4);
                t00[0] = a.x; t00[1] = a.y; t00[2] = a.z; t00[3] = a.w;
                a = *reinterpret_cast<const float4*>(Tb + (16 + ln) * LDM + 16 + g * 4);
                t11[0] = a.x; t11[1] = a.y; t11[2] = a.z; t11[3] = a.w;
                a = *reinterpret_cast<const float4*>(Tb + (16 + ln) * LDM + g * 4);
                nl10[0] = a.x; nl10[1] = a.y; nl10[2] = a.z; nl10[3] = a.w;
                auto subst = [&](const f32x4& r0, const f32x4& r1, f32x4& u0, f32x4& u1) {
                    float b[4];
                    u0 = f32x4{0.f, 0.f, 0.f, 0.f};
                    u1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int r = 0; r < 4; ++r) b[r] = r0[r];
                    mma_k16<F32, SPLITB>(u0, t00, b);
                    f32x4 rhs = r1;
#pragma unroll
                    for (int r = 0; r < 4; ++r) b[r] = u0[r];
                    mma_k16<F32, SPLITB>(rhs, nl10, b);
#pragma unroll
                    for (int r = 0; r < 4; ++r) b[r] = rhs[r];
                    mma_k16<F32, SPLITB>(u1, t11, b);
                };
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) subst(R[0][ct], R[1][ct], U0[ct], U1[ct]);
                if constexpr (DUAL) {
                    // the identity chain (v = 0), after the first one so that
                    // its K+ S, R' and U reuse those registers; its U goes
                    // straight into its B operands
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        Frag<F32> bS[NCT], bSl[NCT];
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) state_op(S2, ks, ct, bS[ct], bSl[ct]);
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb) {
                            Frag<F32> aK;
                            load_tile(aK, sX[buf] + (tb * 16 + ln) * LDR + ks * 32 + g * 4);
#pragma unroll
                            for (int ct = 0; ct < NCT; ++ct) {
                                if constexpr (!F32) mma(R2[tb][ct], aK, bSl[ct]);
                                mma(R2[tb][ct], aK, bS[ct]);
                            }
                        }
                    }
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                            for (int r = 0; r < 4; ++r) R2[tb][ct][r] = -pb[tb][r] * R2[tb][ct][r];
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        f32x4 u0, u1;
                        subst(R2[0][ct], R2[1][ct], u0, u1);
                        float f[8];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            f[r] = u0[r];
                            f[4 + r] = u1[r];
                        }
                        if constexpr (F32) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) bUh2[ct].v[e] = f[e];
                        } else {
                            SplitBF<8> s8 = split8(f);
                            bUh2[ct].v = s8.hi;
                            bUl2[ct].v = s8.lo;
                        }
                    }
                }
            }
            if constexpr (STORE_H) {
                const int64_t cs = t0 + cidx * CH;
                const auto ru = make_rsrc(p.u_out + ((size_t)(cs + srow) * H + h) * DK, span_bytes(n_valid(cs), 4));
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int el = (g * 4 + r) * rowel + col0 + ct * 16 + ln;
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(U0[ct][r]), ru, el * 4, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(U1[ct][r]), ru,
                                                              (el + 16 * rowel) * 4, 0, 0);
                    }
            }
            // U as the B operand of M U and Y^T U (tile order: U0 rows, U1 rows).
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                float f[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    f[r] = U0[ct][r];
                    f[4 + r] = U1[ct][r];
                }
                if constexpr (F32) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) bUh[ct].v[e] = f[e];
                } else {
                    SplitBF<8> s8 = split8(f);
                    bUh[ct].v = s8.hi;
                    bUl[ct].v = s8.lo;
                }
            }
            __syncthreads();
            // ---------------------------------------------------- phase B
            const int64_t c0 = t0 + cidx * CH;
            // O = Q+ S + M U (skipped when o is not wanted); rows past the
            // sequence end fall outside the store range.
            if (!DUAL && p.o) {
                const auto ro = make_rsrc(p.o + ((size_t)c0 * H + h) * DK, span_bytes(n_valid(c0), 4));
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    Frag<F32> aM, aMl;
                    {
                        const uint32_t* mr = sM[buf] + (tb * 16 + ln) * LDM + g * 4;
                        const uint4 m0 = *reinterpret_cast<const uint4*>(mr);
                        const uint4 m1 = *reinterpret_cast<const uint4*>(mr + 16);
                        if constexpr (F32) {
                            aM.v[0] = __uint_as_float(m0.x); aM.v[1] = __uint_as_float(m0.y);
                            aM.v[2] = __uint_as_float(m0.z); aM.v[3] = __uint_as_float(m0.w);
                            aM.v[4] = __uint_as_float(m1.x); aM.v[5] = __uint_as_float(m1.y);
                            aM.v[6] = __uint_as_float(m1.z); aM.v[7] = __uint_as_float(m1.w);
                        } else {
                            uint4 hv, lv;
                            hv.x = perm2(m0.y, m0.x, LO_HALVES); hv.y = perm2(m0.w, m0.z, LO_HALVES);
                            hv.z = perm2(m1.y, m1.x, LO_HALVES); hv.w = perm2(m1.w, m1.z, LO_HALVES);
                            lv.x = perm2(m0.y, m0.x, HI_HALVES); lv.y = perm2(m0.w, m0.z, HI_HALVES);
                            lv.z = perm2(m1.y, m1.x, HI_HALVES); lv.w = perm2(m1.w, m1.z, HI_HALVES);
                            aM.v = __builtin_bit_cast(bf16x8, hv);
                            aMl.v = __builtin_bit_cast(bf16x8, lv);
                        }
                    }
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        if constexpr (!F32) {
                            mma(O[tb][ct], aMl, bUh[ct]);
                            mma(O[tb][ct], aM, bUl[ct]);
                        }
                        mma(O[tb][ct], aM, bUh[ct]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int el = (tb * 16 + g * 4 + r) * rowel + col0 + ct * 16 + ln;
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O[tb][ct][r]), ro,
                                                                  el * 4, 0, 0);
                        }
                    }
                }
            }
            // S <- e^{E1 - E0} (S~ + Y^T U), and, when another chunk follows,
            // already that chunk's S~ (its scan ran in this step's phase A):
            // this phase has slack, the next one does not.
            const float* e1 = sVec[buf][1];
            const bool more = cidx + 1 < nch;
            const float* e0n = sVec[buf ^ 1][0];
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                Frag<F32> aY, aYl;
                load_tile(aY, &sYt[buf][(it * 16 + ln) * LDY + g * 4]);
                if constexpr (!F32) load_tile(aYl, &sYtl[buf][(it * 16 + ln) * LDY + g * 4]);
                const float4 sc4 = *reinterpret_cast<const float4*>(e1 + it * 16 + g * 4);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    if constexpr (!F32) {
                        mma(S[it][ct], aYl, bUh[ct]);
                        mma(S[it][ct], aY, bUl[ct]);
                    }
                    mma(S[it][ct], aY, bUh[ct]);
                    S[it][ct][0] *= sc4.x;
                    S[it][ct][1] *= sc4.y;
                    S[it][ct][2] *= sc4.z;
                    S[it][ct][3] *= sc4.w;
                    if constexpr (DUAL) {
                        if constexpr (!F32) {
                            mma(S2[it][ct], aYl, bUh2[ct]);
                            mma(S2[it][ct], aY, bUl2[ct]);
                        }
                        mma(S2[it][ct], aY, bUh2[ct]);
                        S2[it][ct][0] *= sc4.x;
                        S2[it][ct][1] *= sc4.y;
                        S2[it][ct][2] *= sc4.z;
                        S2[it][ct][3] *= sc4.w;
                    }
                }
                if constexpr (STORE_H) {
                    if (more) {
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct)
                            store_h(hbase + (size_t)(cidx + 1) * H * (DK * DK), it, ct);
                    }
                }
                // two separate scalings: their product alone can underflow
                // (e^{-80} e^{-80}) where the scaled state does not; a select,
                // not a branch, so the matrix-core chains stay interleaved
                float4 n4 = *reinterpret_cast<const float4*>(e0n + it * 16 + g * 4);
                n4.x = more ? n4.x : 1.f;
                n4.y = more ? n4.y : 1.f;
                n4.z = more ? n4.z : 1.f;
                n4.w = more ? n4.w : 1.f;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    S[it][ct][0] *= n4.x;
                    S[it][ct][1] *= n4.y;
                    S[it][ct][2] *= n4.z;
                    S[it][ct][3] *= n4.w;
                    if constexpr (DUAL) {
                        S2[it][ct][0] *= n4.x;
                        S2[it][ct][1] *= n4.y;
                        S2[it][ct][2] *= n4.z;
                        S2[it][ct][3] *= n4.w;
                    }
                }
            }
            __syncthreads();
        }
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
        if constexpr (DUAL) {
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        p.S_T2[sbase + (size_t)(it * 16 + g * 4 + r) * DK + col0 + ct * 16 + ln] =
                            S2[it][ct][r];
        }
    } else {
        load_beta(0, pbp);
        load_scan(0);
        for (int64_t s = 0; s < nch; ++s) {
            // producers: decay scan of chunk s, which also issues the loads of
            // chunk s + 1 (beta first: phase B waits for it, not for the tiles)
            float pbn[2][4];
            load_beta(s + 1, pbn);
            scan((int)(s & 1), s + 1);
            __syncthreads();
            // producers: L, M tiles and the diagonal inverses of chunk s
            const int buf = (int)(s & 1);
            const Op* X = sX[buf];
            const Op* QX = sQX[buf];
            float* Tb = sT[buf];
            uint32_t* Mb = sM[buf];
            if (role == 0) {
                const f32x4 l00 = block(X, X, 0, sY, sY, 0, false);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = g * 4 + r;
                    sL[row * LDM + ln] = ln < row ? pbp[0][r] * l00[r] : 0.f;
                }
                wave_lds_sync();
                // the inverse is this phase's longest dependency chain: let it
                // issue ahead of the other waves on its SIMD
                __builtin_amdgcn_s_setprio(3);
                invert16(sL, Tb, lane);
                __builtin_amdgcn_s_setprio(0);
            } else if (role == 1) {
                const f32x4 l11 = block(X, X, 16, sY, sY, 16, false);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = g * 4 + r;
                    sL[(16 + row) * LDM + 16 + ln] = ln < row ? pbp[1][r] * l11[r] : 0.f;
                }
                wave_lds_sync();
                __builtin_amdgcn_s_setprio(3);
                invert16(sL + 16 * LDM + 16, Tb + 16 * LDM + 16, lane);
                __builtin_amdgcn_s_setprio(0);
            } else {
                // -L10 (beta-scaled) goes where the consumers read it
                auto l10 = [&]() {
                    const f32x4 v = block(X, X, 16, sY, sY, 0, false);
#pragma unroll
                    for (int r = 0; r < 4; ++r) Tb[(16 + g * 4 + r) * LDM + ln] = -pbp[1][r] * v[r];
                };
                auto m10 = [&]() { store_m(Mb, block(QX, sQXl, 16, sY, sYl, 0, true), 16, 0, false); };
                auto m11 = [&]() { store_m(Mb, block(QX, sQXl, 16, sY, sYl, 16, true), 16, 16, true); };
                auto m00 = [&]() { store_m(Mb, block(QX, sQXl, 0, sY, sYl, 0, true), 0, 0, true); };
                if constexpr (NPROD == 8) {
                    if (role == 2) l10();
                    else if (role == 3) m10();
                    else if (role == 4) m11();
                    else if (role == 5) m00();
                } else {
                    if (role == 2) {
                        l10();
                        m10();
                    } else {
                        m11();
                        m00();
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int r = 0; r < 4; ++r) pbp[tb][r] = pbn[tb][r];
        }
        __syncthreads();   // step nch: consumers finish the last chunk
        __syncthreads();
    }
}

// Longest-first order of the packed sequences: order[rank] = sequence, with
// rank = number of sequences that are longer, or as long with a smaller
// index.  O(n^2) comparisons, used only for small n.
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
    // 16 columns per consumer wave (two slices per head) pairs with eight
    // producer waves, 32 columns (one slice) with four.
    dim3 grid((unsigned)(groups * 8 * p.n_slices));
    const bool hs = p.h_states != nullptr;
#define KDA_FWD(T_, W_, P_)                                                                     \
    do {                                                                                        \
        if (hs)                                                                                 \
            hipLaunchKernelGGL((chunk_fwd_kernel<T_, W_, P_, true>), grid, dim3(64 * (4 + P_)), \
                               0, stream, p);                                                   \
        else                                                                                    \
            hipLaunchKernelGGL((chunk_fwd_kernel<T_, W_, P_, false>), grid,                     \
                               dim3(64 * (4 + P_)), 0, stream, p);                              \
    } while (0)
    if (bf16_in) {
        if (wcols == 32) KDA_FWD(__bf16, 32, 4);
        else return launch_chunk_fwd_pipe(p, stream);
    } else {
        if (wcols == 32) KDA_FWD(float, 32, 4);
        else KDA_FWD(float, 16, 8);
    }
#undef KDA_FWD
    return hipGetLastError();
}

hipError_t launch_chunk_fwd_dual(const PrefillParams& prm, bool bf16_in, hipStream_t stream) {
    PrefillParams p = prm;
    p.order = nullptr;
    p.o = nullptr;
    p.s0_identity = 0;
    if (p.n_slices != 1 || !p.S_T || !p.S_T2) return hipErrorInvalidValue;
    const int64_t groups = ((int64_t)p.n_units + 7) / 8;
    const dim3 grid((unsigned)(groups * 8)), block(64 * 8);
    if (bf16_in)
        hipLaunchKernelGGL((chunk_fwd_kernel<__bf16, 32, 4, false, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((chunk_fwd_kernel<float, 32, 4, false, true>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda
