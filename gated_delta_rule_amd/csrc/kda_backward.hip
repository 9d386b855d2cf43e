// Chunkwise KDA backward pass (gfx950).
//
// The pages name the backward kernel (chunk_bwd) as what training needs
// ("尝试对Kimi KDA的数学推导&算子实现分析", the kernel list) but give no formula
// for it; what follows is the reverse-mode derivative of the chunk form the
// forward uses (same page, eqs. (51)-(66), row-beta form).  Per chunk of
// C = 32 tokens with incoming state S, g_t the in-chunk running sum of
// log alpha, G = e^{g} per channel, k+ = k G, q+ = q G, k- = k / G,
// k_end = k e^{g_C - g}:
//   P = StrictTril(K+ K-^T),  A = Diag(beta) P,  T = (I + A)^{-1}
//   M = Tril(Q+ K-^T),  R = V - K+ S,  U = T Diag(beta) R
//   O = Q+ S + M U,  S_next = Diag(e^{g_C}) S + K_end^T U.
// Given dO and Sn = dL/dS_next:
//   dU = M^T dO + K_end Sn,   W = T^T dU          (W = dL/d(Diag(beta) R))
//   dS = Diag(e^{g_C}) Sn + Q+^T dO - K+^T Diag(beta) W
//   dv = Diag(beta) W
//   dM = Tril(dO U^T),  dA' = StrictTril(W U^T)   (dL/dA = -dA')
//   dbeta_t = W_t . R_t - sum_{j<t} dA'_tj P_tj
//   dQ+ = dO S^T + dM K-;   dK+ = -Diag(beta) W S^T - Diag(beta) dA' K-
//   dK- = dM^T Q+ - dA'^T Diag(beta) K+;   dK_end = U Sn^T
// and through the scalings (elementwise, per channel):
//   dq = dQ+ G,  dk = dK+ G + dK- / G + dK_end e^{g_C - g}
//   dg_t = q dq + k (dK+ G - dK- / G - dK_end e^{g_C - g})
//   dg_C += sum_t k dK_end e^{g_C - g} + e^{g_C} rowsum(Sn * S)
//   dlog_alpha_r = sum_{t >= r} dg_t   (within the chunk).
// Products whose factors alone leave the fp32 range (k- = k e^{-g} with g
// down to -160) are formed about the reference E0 = g at the chunk's 16th
// token, as in the forward: X = k e^{g - E0}, Y = k e^{E0 - g},
// Qr = q e^{g - E0}; then P = X Y^T, M = Qr Y^T, dM K- G = (dM Y) e^{g - E0},
// dM^T Q+ / G = (dM^T Qr) e^{E0 - g}, and so on.
//
// MI355X design: three passes after a forward pass that stores the state
// at every chunk start (the prefill kernel with its state output):
//   1. tmp:  one workgroup per (chunk, head), all chunks at once: the decay
//            scan, P and M on the matrix cores, T by forward substitution.
//   2. scan: one workgroup per (sequence, head, 32 value columns) walks the
//            chunks backwards with its 128 x 32 slice of dS in MFMA
//            accumulators (each wave 32 key rows); it writes W, dv and the
//            gradient at every chunk end, and dS0.
//   3. grad: one workgroup per (chunk, head), all chunks at once: every
//            remaining product of the list above from S, Sn, W and the
//            chunk's inputs, then the elementwise chain rule and the
//            in-chunk reverse scan of dg.
// All products run on the fp32 matrix cores (v_mfma_f32_32x32x2f32): a
// wave's 32 x 32 accumulator gives lane l column l % 32 and rows
// 8 (r / 4) + 4 (l / 32) + r % 4 (r = 0..15).  Like the forward, the k order
// of a product is chosen so that accumulators feed the next product's B
// operand without a round trip through LDS.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int BC = 32;        // tokens per chunk
constexpr int BD = 128;       // head dimension
constexpr int LS = BD + 1;    // LDS row stride of [*][128] tiles (odd: rows read across lanes
                              // fall in distinct banks)
constexpr int LC = BC + 1;    // row stride of [32][32] tiles
// Per (chunk, head) matrices from the first pass, in the orders the
// second and third passes read them (floats):
constexpr int OFF_TT = 0;        // T^T            [32][32]
constexpr int OFF_MT = 1024;     // M^T            [32][32]
constexpr int OFF_P = 2048;      // P              [32][32] (strictly lower)
constexpr int OFF_KE = 3072;     // K_end^T        [128][32]
constexpr int OFF_QT = 7168;     // Q+^T           [128][32]
constexpr int OFF_KB = 11264;    // -(B_beta K+)^T [128][32]
constexpr int OFF_GC = 15360;    // e^{g_C}        [128]
constexpr int TMP_ELEMS = 15488;

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mma(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}
// row of accumulator element r in lane l (its column is l % 32)
__device__ __forceinline__ int crow(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <typename InT>
__device__ __forceinline__ float ld_in(const void* base, int64_t idx) {
    return to_f32(reinterpret_cast<const InT*>(base)[idx]);
}

// First token of sequence n (clamped into [0, T] like the forward).
__device__ __forceinline__ int64_t seq_start(const BwdParams& p, int n) {
    if (!p.cu) return (int64_t)n * p.T;
    const int64_t a = p.cu[n];
    return a < 0 ? 0 : (a > p.T ? p.T : a);
}
__device__ __forceinline__ int64_t seq_end(const BwdParams& p, int n, int64_t start) {
    if (!p.cu) return (int64_t)(n + 1) * p.T;
    const int64_t b = p.cu[n + 1];
    return b < start ? start : (b > p.T ? p.T : b);
}

// Chunk held by slot m: chunk j of sequence n uses slot start_n / 32 + n + j
// (strictly increasing in n, so a binary search finds n).  nv = 0: no chunk.
struct Chunk {
    int64_t c0;
    int nv;
};
__device__ Chunk slot_chunk(const BwdParams& p, int64_t m) {
    int lo = 0, hi = p.n_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (seq_start(p, mid) / BC + mid <= m) lo = mid;
        else hi = mid;
    }
    const int64_t s = seq_start(p, lo), e = seq_end(p, lo, s);
    const int64_t j = m - (s / BC + lo);
    Chunk c{s + j * BC, 0};
    if (j >= 0 && c.c0 < e) c.nv = (int)(e - c.c0 < BC ? e - c.c0 : BC);
    return c;
}

// Decay scan of one chunk by 256 threads: thread (channel c = tid % 128,
// half = tid / 128) sums log alpha over tokens 16 half .. 16 half + 15.
// Returns the running sums in g[] (without the other half's offset) and
// leaves both halves' totals in tot[2][128].
__device__ __forceinline__ void chunk_scan(const float* la, int64_t c0, int nv, int H, int h,
                                           int c, int half, float (&g)[16], float* tot) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = 16 * half + i;
        a += t < nv ? la[((c0 + t) * H + h) * BD + c] : 0.f;
        g[i] = a;
    }
    tot[half * BD + c] = a;
}

}  // namespace

// ---------------------------------------------------------------- pass 1
template <typename InT>
__global__ __launch_bounds__(256) void bwd_tmp_kernel(BwdParams p) {
    __shared__ float sX[BC * LS], sY[BC * LS], sQ[BC * LS];   // sX holds A once P is done
    __shared__ float sTot[2 * BD];
    __shared__ float sBeta[BC];
    const int64_t m = blockIdx.x / p.H;
    const int h = (int)(blockIdx.x - m * p.H);
    const Chunk ch = slot_chunk(p, m);
    if (ch.nv == 0) return;
    const int H = p.H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = tid & (BD - 1), half = __builtin_amdgcn_readfirstlane(tid >> 7);
    const int rowb = H * BD * 4;
    const int64_t e0i = (ch.c0 * H + h) * BD;
    const int span = (ch.nv - 1) * rowb + BD * 4;
    constexpr int ES = (int)sizeof(InT);
    const auto rla = make_rsrc(p.la + e0i, span);
    const auto rk = make_rsrc((const InT*)p.k + e0i, span / (4 / ES));
    const auto rq = make_rsrc((const InT*)p.q + e0i, span / (4 / ES));
    const auto rb = make_rsrc(p.beta + ch.c0 * H + h, ((ch.nv - 1) * H + 1) * 4);
    float la[16], kr[16], qr[16], br[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = 16 * half + i;
        // the whole offset in the per-lane operand, so that the range check
        // covers it (rows past the sequence end read as zero)
        la[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rla, t * rowb + c * 4, 0, 0));
        if constexpr (ES == 4) {
            kr[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rk, t * rowb + c * 4, 0, 0));
            qr[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rq, t * rowb + c * 4, 0, 0));
        } else {
            kr[i] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rk, t * (rowb / 2) + c * 2, 0, 0) << 16);
            qr[i] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rq, t * (rowb / 2) + c * 2, 0, 0) << 16);
        }
        br[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, t * H * 4, 0, 0));
    }
    {
        float so = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) so += la[i];
        sTot[half * BD + c] = so;
        if (c == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sBeta[16 * half + i] = br[i];
        }
    }
    lds_barrier();
    float* tmp = p.tmp + ((size_t)m * H + h) * TMP_ELEMS;
    {
        const float E0 = sTot[c];                    // g at token 15
        const float gC = sTot[c] + sTot[BD + c];
        float g = half ? E0 : 0.f;
        float ke[16], qp[16], kb[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 16 * half + i;
            g += la[i];
            const float d = g - E0;
            const float fx = expf(d), fy = expf(-d), G = expf(g);
            sX[t * LS + c] = kr[i] * fx;
            sY[t * LS + c] = kr[i] * fy;
            sQ[t * LS + c] = qr[i] * fx;
            ke[i] = kr[i] * expf(gC - g);
            qp[i] = qr[i] * G;
            kb[i] = -br[i] * kr[i] * G;
        }
        // channel-major rows c of K_end^T, Q+^T, Kb^T (this thread's 16 tokens)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int o = c * BC + 16 * half + 4 * v;
            *reinterpret_cast<float4*>(tmp + OFF_KE + o) =
                make_float4(ke[4 * v], ke[4 * v + 1], ke[4 * v + 2], ke[4 * v + 3]);
            *reinterpret_cast<float4*>(tmp + OFF_QT + o) =
                make_float4(qp[4 * v], qp[4 * v + 1], qp[4 * v + 2], qp[4 * v + 3]);
            *reinterpret_cast<float4*>(tmp + OFF_KB + o) =
                make_float4(kb[4 * v], kb[4 * v + 1], kb[4 * v + 2], kb[4 * v + 3]);
        }
        if (half == 0) tmp[OFF_GC + c] = expf(gC);
    }
    lds_barrier();
    const int i0 = lane & 31, kh = lane >> 5;
    if (wave == 0) {
        // P = StrictTril(X Y^T); A = Diag(beta) P; T = (I + A)^{-1}
        f32x16 acc = zero16();
#pragma unroll 8
        for (int k0 = 0; k0 < BD; k0 += 2)
            acc = mma(sX[i0 * LS + k0 + kh], sY[i0 * LS + k0 + kh], acc);
        float* sA = sX;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = crow(r, lane);
            const float pv = i0 < i ? acc[r] : 0.f;
            tmp[OFF_P + i * BC + i0] = pv;
            sA[i * LC + i0] = sBeta[i] * pv;
        }
        wave_lds_fence();
        if (lane < BC) {
            // column `lane` of T by forward substitution, stored as row `lane` of T^T
            float x[BC];
#pragma unroll
            for (int t = 0; t < BC; ++t) {
                float s = t == lane ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < t; ++j) s -= sA[t * LC + j] * x[j];
                x[t] = s;
            }
#pragma unroll
            for (int v = 0; v < BC / 4; ++v)
                *reinterpret_cast<float4*>(tmp + OFF_TT + lane * BC + 4 * v) =
                    make_float4(x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]);
        }
    } else if (wave == 1) {
        // M = Tril(Qr Y^T), stored transposed
        f32x16 acc = zero16();
#pragma unroll 8
        for (int k0 = 0; k0 < BD; k0 += 2)
            acc = mma(sQ[i0 * LS + k0 + kh], sY[i0 * LS + k0 + kh], acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = crow(r, lane);
            tmp[OFF_MT + i0 * BC + i] = i0 <= i ? acc[r] : 0.f;
        }
    }
}

// ---------------------------------------------------------------- pass 2
// One workgroup of 8 waves per (sequence, head, 64 value columns): wave
// (sw, rw) owns key rows 32 rw .. of value columns 64 sp + 32 sw ..  Per
// chunk, walking backwards:
//   phase 1  part = K_end[:, rows] dS_rows  (+ M^T dO on the rw = 1 waves),
//            QdO = Q+^T dO for its rows;  partial sums to LDS
//   phase 2  (rw = 0) dU = sum of the parts, W = T^T dU, to LDS and memory
//   phase 3  dS = Diag(e^{g_C}) dS + QdO - (B_beta K+)^T W
// Operands are read straight from the first pass's matrices in MFMA order;
// each group is loaded for the next chunk as soon as this chunk's use ends.
template <typename InT>
__global__ __launch_bounds__(512) void bwd_scan_kernel(BwdParams p) {
    __shared__ float sPart[2][4][BC * LC];
    __shared__ float sW[2][BC * LC];

    const int blk = blockIdx.x;
    const int xcd = blk & 7;
    const int grp = blk >> 3;
    const int sp = grp & 1;
    const int unit = (grp >> 1) * 8 + xcd;
    if (unit >= p.n_seqs * p.H) return;
    const int n = unit / p.H, h = unit - n * p.H;
    const int H = p.H;
    const int64_t t0 = seq_start(p, n), t1 = seq_end(p, n, t0);
    const int64_t nch = (t1 - t0 + BC - 1) / BC;
    const int64_t slot0 = t0 / BC + n;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sw = wave >> 2, rw = wave & 3;
    const int i0 = lane & 31, kh = lane >> 5;
    const int col = 64 * sp + 32 * sw + i0;   // this lane's value column
    const int row0 = 32 * rw;                 // this wave's first key row
    const size_t unit_el = ((size_t)n * H + h) * (BD * BD);
    const int rowb = H * BD * 4;

    // Operands, loaded for the next chunk as soon as this chunk's use ends.
    // Group A (phase 1): K_end^T entries, Q+^T row, e^{g_C} of the rows, the
    // dO column and, on the rw = 1 waves, the M^T row.  The T^T row of the
    // rw = 0 waves (phase 2) shares the registers of the M^T row.  Group B
    // (phase 3): the Kb^T row.
    float ke[16], dOr[16];
    float4 qt[4], gc[4], spc[4], kbt[4];
    // buffer loads: one per-lane offset register per operand, the per-load
    // part of the offset in the scalar offset
    auto tmp_rsrc = [&](int64_t j) {
        return make_rsrc(p.tmp + ((size_t)(slot0 + j) * H + h) * TMP_ELEMS, TMP_ELEMS * 4);
    };
    auto ld1 = [](__amdgpu_buffer_rsrc_t r, int vo, int so) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0));
    };
    auto ld4 = [](__amdgpu_buffer_rsrc_t r, int vo, int so) {
        const u32x4 u = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0));
        return make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]),
                           __uint_as_float(u[3]));
    };
    const int vo_ke = ((row0 + 4 * kh) * BC + i0) * 4;   // + (8 (r/4) + r%4) rows
    const int vo_row = ((row0 + i0) * BC + 4 * kh) * 4;  // row row0 + i0 of a [128][32] matrix
    const int vo_sq = (i0 * BC + 4 * kh) * 4;             // row i0 of a [32][32] matrix
    const int vo_gc = (row0 + 4 * kh) * 4;
    auto load_a = [&](int64_t j) {
        const int64_t c0 = t0 + j * BC;
        const int nv = (int)(t1 - c0 < BC ? t1 - c0 : BC);
        const auto rt = tmp_rsrc(j);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            ke[r] = ld1(rt, vo_ke, (OFF_KE + (8 * (r >> 2) + (r & 3)) * BC) * 4);
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            qt[m4] = ld4(rt, vo_row, (OFF_QT + 8 * m4) * 4);
            gc[m4] = ld4(rt, vo_gc, (OFF_GC + 8 * m4) * 4);
            if (rw == 1) spc[m4] = ld4(rt, vo_sq, (OFF_MT + 8 * m4) * 4);
        }
        const auto rdo = make_rsrc(p.dO + (c0 * H + h) * BD, (nv - 1) * rowb + BD * 4);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dOr[r] = ld1(rdo, crow(r, lane) * rowb + col * 4, 0);   // range-checked offset
    };
    auto load_t = [&](int64_t j) {   // rw = 0 waves
        const auto rt = tmp_rsrc(j);
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) spc[m4] = ld4(rt, vo_sq, (OFF_TT + 8 * m4) * 4);
    };
    auto load_b = [&](int64_t j) {
        const auto rt = tmp_rsrc(j);
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) kbt[m4] = ld4(rt, vo_row, (OFF_KB + 8 * m4) * 4);
    };
    auto f4 = [](const float4& v, int s) { return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w; };

    // dS rows row0 + crow(r), column col
    f32x16 dS;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        dS[r] = p.dS_T ? p.dS_T[unit_el + (size_t)(row0 + crow(r, lane)) * BD + col] : 0.f;
    if (nch > 0) {
        load_a(nch - 1);
        if (rw == 0) load_t(nch - 1);
        load_b(nch - 1);
    }

    for (int64_t j = nch - 1; j >= 0; --j) {
        const int64_t c0 = t0 + j * BC;
        const int nv = (int)(t1 - c0 < BC ? t1 - c0 : BC);
        const size_t sl = ((size_t)(slot0 + j) * H + h);
        // gradient at the end of this chunk
        float* dsn = p.dsn + sl * (BD * BD);
#pragma unroll
        for (int r = 0; r < 16; ++r) dsn[(size_t)(row0 + crow(r, lane)) * BD + col] = dS[r];

        // ---- phase 1 (the k order of every product below pairs row / token
        // crow(r, lane) of the two lane halves; r = 4 m4 + s)
        f32x16 part = zero16();
#pragma unroll
        for (int r = 0; r < 16; ++r) part = mma(ke[r], dS[r], part);
        if (rw == 1) {
#pragma unroll
            for (int r = 0; r < 16; ++r) part = mma(f4(spc[r >> 2], r & 3), dOr[r], part);
        }
        // dS <- Diag(e^{g_C}) dS + Q+^T dO
#pragma unroll
        for (int r = 0; r < 16; ++r) dS[r] *= f4(gc[r >> 2], r & 3);
#pragma unroll
        for (int r = 0; r < 16; ++r) dS = mma(f4(qt[r >> 2], r & 3), dOr[r], dS);
#pragma unroll
        for (int r = 0; r < 16; ++r) sPart[sw][rw][crow(r, lane) * LC + i0] = part[r];
        if (j > 0) load_a(j - 1);
        lds_barrier();
        // ---- phase 2: W = T^T dU
        if (rw == 0) {
            f32x16 W = zero16();
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int e = crow(r, lane) * LC + i0;
                const float dU = (sPart[sw][0][e] + sPart[sw][1][e]) + (sPart[sw][2][e] + sPart[sw][3][e]);
                W = mma(f4(spc[r >> 2], r & 3), dU, W);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = crow(r, lane);
                sW[sw][t * LC + i0] = W[r];
                if (t < nv) p.w[((size_t)(c0 + t) * H + h) * BD + col] = W[r];
            }
            if (j > 0) load_t(j - 1);
        }
        lds_barrier();
        // ---- phase 3: dS <- dS - (B_beta K+)^T W
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dS = mma(f4(kbt[r >> 2], r & 3), sW[sw][crow(r, lane) * LC + i0], dS);
        if (j > 0) load_b(j - 1);
    }
    if (p.dS0) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            p.dS0[unit_el + (size_t)(row0 + crow(r, lane)) * BD + col] = dS[r];
    }
}

// ---------------------------------------------------------------- pass 3
template <typename InT>
__global__ __launch_bounds__(256) void bwd_grad_kernel(BwdParams p) {
    __shared__ float sS[BD * LS];      // S, then Sn, then g
    __shared__ float sA1[BC * LS];     // K+, then X, then dg
    __shared__ float sA2[BC * LS];     // dO, then Y
    __shared__ float sA3[BC * LS];     // W, then Qr
    __shared__ float sU[BC * LS];      // U, then g
    __shared__ float sT[BC * LC];
    __shared__ float sdM[BC * LC], sdA[BC * LC];
    __shared__ float sTot[2 * BD];
    __shared__ float sRow[BD], sGx[BD];
    __shared__ float sBeta[BC];
    __shared__ float sDb[5][BC];

    const int64_t m = blockIdx.x / p.H;
    const int h = (int)(blockIdx.x - m * p.H);
    const Chunk ch = slot_chunk(p, m);
    if (ch.nv == 0) return;
    const int H = p.H, nv = ch.nv;
    const int64_t c0 = ch.c0;
    const size_t sl = (size_t)m * H + h;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = tid & (BD - 1), half = tid >> 7;
    const int i0 = lane & 31, kh = lane >> 5;

    // ---- phase 0: loads
    float g[16], kv[16], qv[16];
    chunk_scan(p.la, c0, nv, H, h, c, half, g, sTot);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = 16 * half + i;
        const int64_t idx = ((c0 + t) * H + h) * BD + c;
        kv[i] = t < nv ? ld_in<InT>(p.k, idx) : 0.f;
        qv[i] = t < nv ? ld_in<InT>(p.q, idx) : 0.f;
    }
    if (tid < BC) sBeta[tid] = tid < nv ? p.beta[(c0 + tid) * H + h] : 0.f;
    {
        const float* hs = p.h + sl * (BD * BD);
#pragma unroll 4
        for (int e = 0; e < 16; ++e) {
            const int idx = (tid + 256 * e) * 4;   // float4 index * 4
            const int r = idx >> 7, cc = idx & 127;
            const float4 v4 = *reinterpret_cast<const float4*>(hs + idx);
            sS[r * LS + cc] = v4.x;
            sS[r * LS + cc + 1] = v4.y;
            sS[r * LS + cc + 2] = v4.z;
            sS[r * LS + cc + 3] = v4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = (tid + 256 * e) * 4;
            const int r = idx >> 7, cc = idx & 127;
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
            if (r < nv) {
                const size_t o = ((size_t)(c0 + r) * H + h) * BD + cc;
                a = *reinterpret_cast<const float4*>(p.dO + o);
                b = *reinterpret_cast<const float4*>(p.w + o);
                const float bt = p.beta[(c0 + r) * H + h];   // dv = beta W
                *reinterpret_cast<float4*>(p.dv + o) = make_float4(bt * b.x, bt * b.y, bt * b.z, bt * b.w);
            }
            sA2[r * LS + cc] = a.x; sA2[r * LS + cc + 1] = a.y;
            sA2[r * LS + cc + 2] = a.z; sA2[r * LS + cc + 3] = a.w;
            sA3[r * LS + cc] = b.x; sA3[r * LS + cc + 1] = b.y;
            sA3[r * LS + cc + 2] = b.z; sA3[r * LS + cc + 3] = b.w;
        }
        const float* tm = p.tmp + sl * TMP_ELEMS + OFF_TT;   // T^T
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = tid + 256 * e;
            sT[(idx & 31) * LC + (idx >> 5)] = tm[idx];
        }
    }
    lds_barrier();
    const float e0 = sTot[c];
    const float gC = sTot[c] + sTot[BD + c];
    const float off = half ? e0 : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = 16 * half + i;
        sA1[t * LS + c] = kv[i] * expf(g[i] + off);   // K+ (may underflow: only ever small)
    }
    lds_barrier();

    // ---- phase 1: R = V - K+ S, dbeta (first part), U = T Diag(beta) R
    const int vcol = 32 * wave + i0;   // value column (phase 1) / key column (later)
    f32x16 U;
    {
        f32x16 R = zero16();
#pragma unroll 8
        for (int k0 = 0; k0 < BD; k0 += 2)
            R = mma(sA1[i0 * LS + k0 + kh], sS[(k0 + kh) * LS + vcol], R);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = crow(r, lane);
            const float vv = t < nv ? ld_in<InT>(p.v, ((c0 + t) * H + h) * BD + vcol) : 0.f;
            R[r] = vv - R[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float s = half_sum_dpp(sA3[crow(r, lane) * LS + vcol] * R[r]);
            if (i0 == 0) sDb[wave][crow(r, lane)] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) R[r] *= sBeta[crow(r, lane)];
        U = zero16();
#pragma unroll
        for (int r = 0; r < 16; ++r) U = mma(sT[i0 * LC + crow(r, lane)], R[r], U);
#pragma unroll
        for (int r = 0; r < 16; ++r) sU[crow(r, lane) * LS + vcol] = U[r];
    }
    lds_barrier();

    // ---- phase 2: dM = dO U^T (waves 0, 1), dA' = W U^T (waves 2, 3), each
    // pair splitting the value columns; X1 = dO S^T, X2 = W S^T for key
    // columns 32 wave ..
    f32x16 X1 = zero16(), X2 = zero16(), CC = zero16();
    {
        const float* Ain = wave < 2 ? sA2 : sA3;
        const int kb = (wave & 1) * 64;
#pragma unroll 8
        for (int k0 = 0; k0 < 64; k0 += 2)
            CC = mma(Ain[i0 * LS + kb + k0 + kh], sU[i0 * LS + kb + k0 + kh], CC);
        if (wave & 1) {
            float* dst = wave == 1 ? sdM : sdA;
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[crow(r, lane) * LC + i0] = CC[r];
        }
#pragma unroll 8
        for (int k0 = 0; k0 < BD; k0 += 2) {
            const float b = sS[vcol * LS + k0 + kh];
            X1 = mma(sA2[i0 * LS + k0 + kh], b, X1);
            X2 = mma(sA3[i0 * LS + k0 + kh], b, X2);
        }
    }
    lds_barrier();

    // ---- phase 3: finish dM / dA'; Sn over S with rowsum(Sn * S); X, Y, Qr
    if (!(wave & 1)) {
        float* dst = wave == 0 ? sdM : sdA;
        const float* P = p.tmp + sl * TMP_ELEMS + OFF_P;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = crow(r, lane);
            const float v = CC[r] + dst[i * LC + i0];
            if (wave == 0) {
                dst[i * LC + i0] = i0 <= i ? v : 0.f;                       // dM
            } else {
                const float da = i0 < i ? v : 0.f;                          // dA'
                dst[i * LC + i0] = -sBeta[i] * da;                          // dPm
                const float s = half_sum_dpp(-da * P[i * BC + i0]);
                if (i0 == 0) sDb[4][i] = s;
            }
        }
    }
    {
        const float* sn = p.dsn + sl * (BD * BD);
        const int r = tid >> 1, cb = (tid & 1) * 64;
        float acc = 0.f;
#pragma unroll 4
        for (int e = 0; e < 16; ++e) {
            const float4 v4 = *reinterpret_cast<const float4*>(sn + r * BD + cb + 4 * e);
            float* d = &sS[r * LS + cb + 4 * e];
            acc += v4.x * d[0] + v4.y * d[1] + v4.z * d[2] + v4.w * d[3];
            d[0] = v4.x; d[1] = v4.y; d[2] = v4.z; d[3] = v4.w;
        }
        acc += dpp_mov<0xB1>(acc);   // partner thread tid ^ 1 holds the other half row
        if (!(tid & 1)) sRow[r] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = 16 * half + i;
        const float d = g[i] + off - e0;
        const float fx = expf(d), fy = expf(-d);
        sA1[t * LS + c] = kv[i] * fx;
        sA2[t * LS + c] = kv[i] * fy;
        sA3[t * LS + c] = qv[i] * fx;
    }
    lds_barrier();

    // ---- phase 4: X3 = U Sn^T, Y1 = dM Y, Y2 = dPm Y, Y34 = dM^T Qr + dPm^T X
    f32x16 X3 = zero16(), Y1 = zero16(), Y2 = zero16(), Y34 = zero16();
#pragma unroll 8
    for (int k0 = 0; k0 < BD; k0 += 2)
        X3 = mma(sU[i0 * LS + k0 + kh], sS[vcol * LS + k0 + kh], X3);
#pragma unroll
    for (int k0 = 0; k0 < BC; k0 += 2) {
        const int t = k0 + kh;
        const float y = sA2[t * LS + vcol];
        Y1 = mma(sdM[i0 * LC + t], y, Y1);
        Y2 = mma(sdA[i0 * LC + t], y, Y2);
        Y34 = mma(sdM[t * LC + i0], sA3[t * LS + vcol], Y34);
        Y34 = mma(sdA[t * LC + i0], sA1[t * LS + vcol], Y34);
    }
    lds_barrier();
    // g (with the half offset) for the elementwise phase
#pragma unroll
    for (int i = 0; i < 16; ++i) sU[(16 * half + i) * LS + c] = g[i] + off;
    lds_barrier();

    // ---- phase 5: chain rule through the scalings, per (token, key column)
    {
        const float E0 = sTot[vcol], GC = sTot[vcol] + sTot[BD + vcol];
        float colsum = 0.f;
        float dgv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = crow(r, lane);
            const float gt = sU[t * LS + vcol];
            const float G = expf(gt), Gr = expf(gt - E0), Gri = expf(E0 - gt), Ge = expf(GC - gt);
            const int64_t idx = ((c0 + t) * H + h) * BD + vcol;
            const float kf = t < nv ? ld_in<InT>(p.k, idx) : 0.f;
            const float qf = t < nv ? ld_in<InT>(p.q, idx) : 0.f;
            const float dq = X1[r] * G + Y1[r] * Gr;
            const float dkp = -sBeta[t] * X2[r] * G + Y2[r] * Gr;
            const float dkm = Y34[r] * Gri;
            const float dke = X3[r] * Ge;
            dgv[r] = qf * dq + kf * (dkp - dkm - dke);
            colsum += kf * dke;
            if (t < nv) {
                p.dq[idx] = dq;
                p.dk[idx] = dkp + dkm + dke;
            }
        }
        colsum += swap_halves(colsum);
#pragma unroll
        for (int r = 0; r < 16; ++r) sA1[crow(r, lane) * LS + vcol] = dgv[r];
        if (kh == 0) sGx[vcol] = colsum + expf(GC) * sRow[vcol];
    }
    lds_barrier();
    if (tid < BD) {
        // dlog_alpha_r = sum_{t >= r} dg_t + dg_C, over the chunk's tokens
        float run = sGx[tid];
        for (int t = nv - 1; t >= 0; --t) {
            run += sA1[t * LS + tid];
            p.dla[((c0 + t) * H + h) * BD + tid] = run;
        }
    } else if (tid < BD + BC) {
        const int t = tid - BD;
        if (t < nv)
            p.dbeta[(c0 + t) * H + h] =
                ((sDb[0][t] + sDb[1][t]) + (sDb[2][t] + sDb[3][t])) + sDb[4][t];
    }
}

hipError_t launch_chunk_bwd(const BwdParams& p, bool bf16_in, hipStream_t stream) {
    const int64_t chunks = p.slots * p.H;
    const int64_t units = (int64_t)p.n_seqs * p.H;
    if (chunks > 0) {
        if (bf16_in) hipLaunchKernelGGL(bwd_tmp_kernel<__bf16>, dim3((unsigned)chunks), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL(bwd_tmp_kernel<float>, dim3((unsigned)chunks), dim3(256), 0, stream, p);
    }
    if (units > 0) {
        const dim3 grid((unsigned)(((units + 7) / 8) * 8 * 2));
        if (bf16_in) hipLaunchKernelGGL(bwd_scan_kernel<__bf16>, grid, dim3(512), 0, stream, p);
        else hipLaunchKernelGGL(bwd_scan_kernel<float>, grid, dim3(512), 0, stream, p);
    }
    if (chunks > 0) {
        if (bf16_in) hipLaunchKernelGGL(bwd_grad_kernel<__bf16>, dim3((unsigned)chunks), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL(bwd_grad_kernel<float>, dim3((unsigned)chunks), dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace kda
