// Chunkwise KDA prefill for bf16 inputs, three-stage pipeline (gfx950).
//
// Same algebra, chunking (C = 32), factoring about E0 and rounding plan as
// chunk_fwd_kernel ("尝试对Kimi KDA的数学推导&算子实现分析" eqs. (51)-(66)):
//   X = k e^{g-E0}, QX = q e^{g-E0}, Y = k e^{E0-g};  L = StrictTril(B X Y^T),
//   M = Tril(QX Y^T),  U = (I + L)^{-1} B (V - X S~),  O = QX S~ + M U,
//   S <- e^{E1-E0} (S~ + Y^T U),  S~ = e^{E0} S.
// What differs is the schedule.  A workgroup of 12 waves (one of each kind
// per SIMD) serves one (sequence, head, 64-column slice); the three kinds of
// wave work on three different chunks between two consecutive workgroup
// barriers, with one barrier per chunk:
//   * scan waves     (4): decay scan of chunk c+2 -> X, QX (hi, lo), Y (hi,
//                         lo), e^{E0}, e^{E1-E0};
//   * tile waves     (4): chunk c+1 -> L blocks, the two 16 x 16 inverses,
//                         -L10 and M (hi, lo);
//   * consumer waves (4): the state-dependent chain of chunk c (16 value
//                         columns each, the state in accumulator registers).
// No wave waits inside a step for another kind's work of the same step, so
// the vector-heavy scan, the latency-bound inverses and the matrix-core
// chain overlap on every SIMD.  Tiles live until their last reader:
// X, QX, Y, Y lo and the scalings three steps, QX lo and the tile waves'
// outputs two.  The state update's Y^T operand is read straight from the
// token-major Y with the gfx950 transposing LDS read, so no transposed copy
// is kept.
#include "kda_chunk.h"
#include "kda_launch.h"

#ifndef KDA_PIPE_NSCAN
#define KDA_PIPE_NSCAN 4
#endif

namespace kda {

namespace {

constexpr int PLDR = DK + 8;   // token-major bf16 row stride
constexpr int LDMB = CH + 8;   // row stride of bf16 [CH][CH] tiles

// One lane's 8 k-values (tokens 4g..4g+3 and 16+4g..16+4g+3, "tile order")
// of the A operand Y^T[key0 + ln][token] from a token-major [CH][PLDR] tile.
// The transposing read hands lane (group g, position i) element i & 3 of
// the 4-element row segment addressed by lane 4j + (i >> 2) of its group as
// its element j, so lane 4j + q addresses token 4g + j, keys key0 + 4q..+3:
// `p` is the tile plus that lane offset, (4g + (ln >> 2)) * PLDR + 4 (ln & 3).
// `a` is the LDS byte address of the tile plus that lane offset.  (The
// transposing read's builtin does not fold constant offsets into the
// instruction, so the address arithmetic is kept to one add per read.)
__device__ __forceinline__ bf16x8 load_tr(uint32_t a, int key0) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef short v8s __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(uintptr_t)(a + 2 * key0));
    const v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(uintptr_t)(a + 2 * (key0 + 16 * PLDR)));
    const v8s c = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return __builtin_bit_cast(bf16x8, c);
}
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Two floats to a packed fp16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    f16x2 r;
    r[0] = (_Float16)a;
    r[1] = (_Float16)b;
    uint32_t u = __builtin_bit_cast(uint32_t, r);
    asm("" : "+v"(u));
    return u;
}
__device__ __forceinline__ f32x4 mfma32h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 8 fp16 values in tile order (p[0..3], p[16..19]).
__device__ __forceinline__ f16x8 load_tile_h(const uint16_t* p) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    const uint2 b = *reinterpret_cast<const uint2*>(p + 16);
    const uint4 v = make_uint4(a.x, a.y, b.x, b.y);
    return __builtin_bit_cast(f16x8, v);
}
// LDS byte address of an element of a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const __bf16* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) __bf16*)p;
}

}  // namespace

// WANT_O: form o (Q+ S and M U); the passes that only need states or the
// backward's per-chunk values skip Q+ S, q e^{g}, QX and M altogether.
// STORE_H: also store, per chunk, the state at its start (h_states), V - K+ S
// (r_out) and U (u_out), as chunk_fwd_kernel does for the backward pass.
template <int NSCAN, bool STORE_H, bool WANT_O, bool SEG>
__global__ __launch_bounds__(64 * (8 + NSCAN)) void chunk_fwd_pipe_kernel(PrefillParams p) {
    constexpr int WCOLS = 16;         // value columns per consumer wave
    constexpr int DVW = 4 * WCOLS;    // value columns per workgroup
    constexpr int LDR = PLDR;
    typedef Frag<false> Fr;

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
    } else if constexpr (SEG) {
        // a first segment of its own length (seg_first, seg_r0)
        const int64_t b = n / p.seg_per_seq;
        const int64_t r = p.seg_r0 + (n - b * p.seg_per_seq);
        const int64_t len = r == 0 ? p.seg_first : p.seg_len;
        const int64_t e = (b + 1) * Tt;
        t0 = b * Tt + (r == 0 ? 0 : p.seg_first + (r - 1) * p.seg_len);
        t0 = t0 < e ? t0 : e;
        t1 = e - t0 > len ? t0 + len : e;
    } else {
        const int64_t b = p.seg_sel >= 0 ? n : n / p.seg_per_seq;
        const int64_t r = p.seg_sel >= 0 ? p.seg_sel : n - b * p.seg_per_seq;
        const int64_t e = (b + 1) * Tt;
        t0 = b * Tt + r * p.seg_len;
        t0 = t0 < e ? t0 : e;
        t1 = e - t0 > p.seg_len ? t0 + p.seg_len : e;
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
    // 0 consumer, 1 scan, 2 tiles; waves 0-3 consumers, then NSCAN scan waves
    const int kind = wave < 4 ? 0 : (wave < 4 + NSCAN ? 1 : 2);
    const int role = kind == 1 ? wave - 4 : (wave & 3);   // column block / scan part / tile role
    const int g = lane >> 4;      // lane group
    const int ln = lane & 15;     // row / column within a 16-wide tile

    // ------------------------------------------------------------------ LDS
    // [c % 3]: written by the scan at step c - 2, read up to step c.
    // [c & 1]: written at step c - 2 or c - 1, read up to step c.
    __shared__ __attribute__((aligned(16))) __bf16 sX[3][CH * LDR];    // k e^{g - E0}
    __shared__ __attribute__((aligned(16))) __bf16 sQX[2][CH * LDR];   // q e^{g - E0} (hi)
    __shared__ __attribute__((aligned(16))) __bf16 sY[3][CH * LDR];    // k e^{E0 - g} (hi)
    __shared__ __attribute__((aligned(16))) __bf16 sYl[3][CH * LDR];   // (lo)
    __shared__ __attribute__((aligned(16))) __bf16 sQXl[2][CH * LDR];  // (lo)
    __shared__ __attribute__((aligned(16))) float sVec[3][2][DK];      // e^{E0}, e^{E1 - E0}
    __shared__ __attribute__((aligned(16))) uint16_t sQp[3][CH * LDR];  // q e^{g} (fp16)
    __shared__ __attribute__((aligned(16))) float sT[2][CH * LDM];     // T00, T11, -L10 (beta-scaled)
    __shared__ __attribute__((aligned(16))) __bf16 sMh[2][CH * LDMB];  // M (hi)
    __shared__ __attribute__((aligned(16))) __bf16 sMl[2][CH * LDMB];  // M (lo)

    // M's upper-right 16 x 16 block is identically zero; never rewritten.
    if (tid < 512) {
        const int e = ((tid & 255) >> 4) * LDMB + 16 + (tid & 15);
        sMh[tid >> 8][e] = (__bf16)0.f;
        sMl[tid >> 8][e] = (__bf16)0.f;
    }

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

    // 16 x 16 block of A B^T over the 128 channels (contiguous k order);
    // with `split`: A B^T = Ah Bh^T + Ah Bl^T + Al Bh^T.
    auto block = [&](const __bf16* A, const __bf16* Al, int arow0, const __bf16* B, const __bf16* Bl,
                     int brow0, bool split) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ao = (arow0 + ln) * LDR + ks * 32 + g * 8;
            const int bo = (brow0 + ln) * LDR + ks * 32 + g * 8;
            Fr a, b;
            load_contig(a, A + ao);
            load_contig(b, B + bo);
            if (split) {
                Fr al, bl;
                load_contig(al, Al + ao);
                load_contig(bl, Bl + bo);
                mma(acc, al, b);
                mma(acc, a, bl);
            }
            mma(acc, a, b);
        }
        return acc;
    };
    // Two split blocks A B1^T and A B2^T that share the A rows (loaded once).
    auto block2 = [&](const __bf16* A, const __bf16* Al, int arow0, const __bf16* B, const __bf16* Bl,
                      int brow1, int brow2, f32x4& acc1, f32x4& acc2) {
        acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
        acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ao = (arow0 + ln) * LDR + ks * 32 + g * 8;
            const int bo1 = (brow1 + ln) * LDR + ks * 32 + g * 8;
            const int bo2 = (brow2 + ln) * LDR + ks * 32 + g * 8;
            Fr a, al, b1, b1l, b2, b2l;
            load_contig(a, A + ao);
            load_contig(al, Al + ao);
            load_contig(b1, B + bo1);
            load_contig(b1l, Bl + bo1);
            load_contig(b2, B + bo2);
            load_contig(b2l, Bl + bo2);
            mma(acc1, al, b1);
            mma(acc2, al, b2);
            mma(acc1, a, b1l);
            mma(acc2, a, b2l);
            mma(acc1, a, b1);
            mma(acc2, a, b2);
        }
    };
    // Store an M block (C layout) at rows r0, columns c0 as hi and lo bf16
    // tiles, keeping j <= t if diag.
    auto store_m = [&](__bf16* Mh, __bf16* Ml, const f32x4& m, int r0, int c0, bool diag) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float v = (!diag || ln <= g * 4 + r) ? m[r] : 0.f;
            const __bf16 hi = (__bf16)v;
            Mh[(r0 + g * 4 + r) * LDMB + c0 + ln] = hi;
            Ml[(r0 + g * 4 + r) * LDMB + c0 + ln] = (__bf16)(v - (float)hi);
        }
    };

    // One barrier per step; step s runs the scan of chunk s + 2, the tiles of
    // chunk s + 1 and the chain of chunk s.  Every kind loops over the same
    // steps, so the barrier counts match.
    if (kind == 0) {
        // ==================================================== consumers
        const int col0 = slice * DVW + role * WCOLS;   // first value column
        f32x4 S[8];
        const size_t sbase = ((size_t)n * H + h) * (DK * DK);
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[it][r] = p.s0_identity ? (it * 16 + g * 4 + r == col0 + ln ? 1.f : 0.f)
                           : p.S0       ? p.S0[sbase + (size_t)(it * 16 + g * 4 + r) * DK + col0 + ln]
                                        : 0.f;
        // v (raw bf16 bits, converted where used) and beta of the next chunk
        uint16_t pv[2][4];
        float pb[2][4];
        auto load_v = [&](int64_t cidx) {
            const int64_t c = t0 + cidx * CH;
            const int nv = n_valid(c);
            const auto rv = make_rsrc((const __bf16*)p.v + ((size_t)c * H + h) * DK,
                                      p.s0_identity ? 0 : span_bytes(nv, 2));
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int el = (tb * 16 + g * 4 + r) * rowel + col0 + ln;
                    pv[tb][r] = __builtin_amdgcn_raw_buffer_load_b16(rv, el * 2, 0, 0);
                }
        };
        // lane offsets (elements) of the operand reads
        const int aoff = ln * LDR + g * 4;                                  // X, QX tile rows
        const int troff = (4 * g + (ln >> 2)) * LDR + 4 * (ln & 3);         // transposed Y reads
        load_v(0);
        load_beta(0, pb);
        for (int64_t s = -2; s < nch; ++s) {
            if (s >= 0) {
                const int b3 = (int)(s % 3), b2 = (int)(s & 1);
                const float* Tb = sT[b2];
                float4 t00v, t11v, l10v;
                if constexpr (STORE_H) {   // the state at this chunk's start -> slot hslot0 + s
                    float* hb = p.h_states + ((size_t)(hslot0 + s) * H + h) * (DK * DK);
#pragma unroll
                    for (int it = 0; it < 8; ++it)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            hb[(size_t)(it * 16 + g * 4 + r) * DK + col0 + ln] = S[it][r];
                }
                // K+ S = X (e^{E0} S) on bf16 matrix cores with the scaled
                // state's hi part (the delta rule corrects that rounding), and
                // Q+ S with both operands in fp16 (q e^{g} <= |q|, so in range):
                // per k-slice the state is packed to fp16, then scaled to
                // S~ = e^{E0} S in place (the update adds to S~) and packed to
                // bf16; the next k-slice's operands load meanwhile.
                f32x4 R[2], O[2];
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    R[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                    O[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                const __bf16* Xb = sX[b3] + aoff;
                const uint16_t* Qb = sQp[b3] + aoff;
                const float* e0 = sVec[b3][0] + g * 4;
                Fr aK[2][2];
                f16x8 aQ[2][2];   // [slot][tb]
                float4 ev[2][2];  // e^{E0} rows of the slice's two state tiles
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    load_tile(aK[0][tb], Xb + tb * 16 * LDR);
                    if constexpr (WANT_O) aQ[0][tb] = load_tile_h(Qb + tb * 16 * LDR);
                    ev[0][tb] = *reinterpret_cast<const float4*>(e0 + tb * 16);
                }
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int cur = ks & 1;
                    if (ks < 3) {
#pragma unroll
                        for (int tb = 0; tb < 2; ++tb) {
                            load_tile(aK[cur ^ 1][tb], Xb + tb * 16 * LDR + (ks + 1) * 32);
                            if constexpr (WANT_O)
                                aQ[cur ^ 1][tb] = load_tile_h(Qb + tb * 16 * LDR + (ks + 1) * 32);
                            ev[cur ^ 1][tb] = *reinterpret_cast<const float4*>(e0 + (2 * ks + 2 + tb) * 16);
                        }
                    }
                    f16x8 bS16;
                    Fr bS;
                    {
                        if constexpr (WANT_O) {
                            u32x4 w;
#pragma unroll
                            for (int i = 0; i < 2; ++i) {
                                w[2 * i] = pack_h2(S[2 * ks + i][0], S[2 * ks + i][1]);
                                w[2 * i + 1] = pack_h2(S[2 * ks + i][2], S[2 * ks + i][3]);
                            }
                            bS16 = __builtin_bit_cast(f16x8, w);
                        }
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            const float4 sc4 = ev[cur][i];
                            S[2 * ks + i][0] *= sc4.x;
                            S[2 * ks + i][1] *= sc4.y;
                            S[2 * ks + i][2] *= sc4.z;
                            S[2 * ks + i][3] *= sc4.w;
                        }
                        float f[8];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            f[r] = S[2 * ks][r];
                            f[4 + r] = S[2 * ks + 1][r];
                        }
                        bS.v = round8(f);
                    }
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) {
                        mma(R[tb], aK[cur][tb], bS);
                        if constexpr (WANT_O) O[tb] = mfma32h(aQ[cur][tb], bS16, O[tb]);
                    }
                    // keep the next slice's loads ahead of this slice's products
                    __builtin_amdgcn_sched_barrier(0);
                }
                t00v = *reinterpret_cast<const float4*>(Tb + ln * LDM + g * 4);
                t11v = *reinterpret_cast<const float4*>(Tb + (16 + ln) * LDM + 16 + g * 4);
                l10v = *reinterpret_cast<const float4*>(Tb + (16 + ln) * LDM + g * 4);
                // R' = B_beta (V - K+ S)  (V - K+ S itself kept for the backward pass)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        R[tb][r] = __uint_as_float((uint32_t)pv[tb][r] << 16) - R[tb][r];
                if constexpr (STORE_H) {
                    const int64_t cs = t0 + s * CH;
                    const auto rr = make_rsrc(p.r_out + ((size_t)(cs + srow) * H + h) * DK, span_bytes(n_valid(cs), 4));
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int el = (tb * 16 + g * 4 + r) * rowel + col0 + ln;
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(R[tb][r]), rr, el * 4, 0, 0);
                        }
                }
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) R[tb][r] *= pb[tb][r];
                // next chunk's values and beta
                load_v(s + 1);
                load_beta(s + 1, pb);
                Fr aM[2], aMl[2];
                if constexpr (WANT_O) {
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) {
                        load_tile(aM[tb], sMh[b2] + (tb * 16 + ln) * LDMB + g * 4);
                        load_tile(aMl[tb], sMl[b2] + (tb * 16 + ln) * LDMB + g * 4);
                    }
                }
                // Block forward substitution of (I + L) U = R':
                //   U0 = T00 R'0,  U1 = T11 (R'1 - L10 U0)
                f32x4 U0, U1;
                {
                    const float t00[4] = {t00v.x, t00v.y, t00v.z, t00v.w};
                    const float t11[4] = {t11v.x, t11v.y, t11v.z, t11v.w};
                    const float nl10[4] = {l10v.x, l10v.y, l10v.z, l10v.w};
                    float b[4];
                    U0 = f32x4{0.f, 0.f, 0.f, 0.f};
                    U1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int r = 0; r < 4; ++r) b[r] = R[0][r];
                    mma_k16<false, SPLITB>(U0, t00, b);
                    f32x4 rhs = R[1];
#pragma unroll
                    for (int r = 0; r < 4; ++r) b[r] = U0[r];
                    mma_k16<false, SPLITB>(rhs, nl10, b);
#pragma unroll
                    for (int r = 0; r < 4; ++r) b[r] = rhs[r];
                    mma_k16<false, SPLITB>(U1, t11, b);
                }
                if constexpr (STORE_H) {
                    const int64_t cs = t0 + s * CH;
                    const auto ru = make_rsrc(p.u_out + ((size_t)(cs + srow) * H + h) * DK, span_bytes(n_valid(cs), 4));
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int el = (g * 4 + r) * rowel + col0 + ln;
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(U0[r]), ru, el * 4, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(U1[r]), ru, (el + 16 * rowel) * 4, 0, 0);
                    }
                }
                // U as the B operand of M U and Y^T U (tile order: U0 rows, U1 rows).
                Fr bUh, bUl;
                {
                    float f[8];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        f[r] = U0[r];
                        f[4 + r] = U1[r];
                    }
                    SplitBF<8> s8 = split8(f);
                    bUh.v = s8.hi;
                    bUl.v = s8.lo;
                }
                // O = Q+ S + M U (skipped when o is not wanted); rows past the
                // sequence end fall outside the store range.
                if (WANT_O && p.o) {
                    const int64_t c0 = t0 + s * CH;
                    const auto ro = make_rsrc(p.o + ((size_t)c0 * H + h) * DK, span_bytes(n_valid(c0), 4));
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) {
                        mma(O[tb], aMl[tb], bUh);
                        mma(O[tb], aM[tb], bUl);
                        mma(O[tb], aM[tb], bUh);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int el = (tb * 16 + g * 4 + r) * rowel + col0 + ln;
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O[tb][r]), ro, el * 4, 0, 0);
                        }
                    }
                }
                // S <- e^{E1 - E0} (S~ + Y^T U): the unscaled state at the chunk
                // end.  The operands of tile it + 1 load while tile it's products
                // issue; tile it - 1 is scaled meanwhile.
                const uint32_t Yb = lds_addr(sY[b3] + troff);
                const uint32_t Ylb = lds_addr(sYl[b3] + troff);
                const float* e1 = sVec[b3][1] + g * 4;
                bf16x8 aY[2], aYl[2];
                aY[0] = load_tr(Yb, 0);
                aYl[0] = load_tr(Ylb, 0);
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    const int cur = it & 1;
                    if (it < 7) {
                        aY[cur ^ 1] = load_tr(Yb, (it + 1) * 16);
                        aYl[cur ^ 1] = load_tr(Ylb, (it + 1) * 16);
                    }
                    S[it] = mfma32(aYl[cur], bUh.v, S[it]);
                    S[it] = mfma32(aY[cur], bUl.v, S[it]);
                    S[it] = mfma32(aY[cur], bUh.v, S[it]);
                    if (it > 0) {
                        const float4 a4 = *reinterpret_cast<const float4*>(e1 + (it - 1) * 16);
                        S[it - 1][0] *= a4.x;
                        S[it - 1][1] *= a4.y;
                        S[it - 1][2] *= a4.z;
                        S[it - 1][3] *= a4.w;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                {
                    const float4 a4 = *reinterpret_cast<const float4*>(e1 + 7 * 16);
                    S[7][0] *= a4.x;
                    S[7][1] *= a4.y;
                    S[7][2] *= a4.z;
                    S[7][3] *= a4.w;
                }
            }
            __syncthreads();
        }
        if (p.S_T) {
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.S_T[sbase + (size_t)(it * 16 + g * 4 + r) * DK + col0 + ln] = S[it][r];
        }
    } else if (kind == 1) {
        // ==================================================== scan waves
        // A wave covers 16 channel pairs for the whole chunk: lane l handles
        // the 8 consecutive tokens 8 (l >> 4) .. of the pair (2 cp, 2 cp + 1),
        // cp = 16 role + (l & 15), so every lane learns the decay E0 after the
        // first 16 tokens from the cross-lane scan.
        static_assert(NSCAN == 4, "one scan wave per SIMD");
        constexpr int TPL = 8;
        const int cp = role * 16 + (lane & 15);
        const int part = lane >> 4;
        const int sc = 2 * cp;
        uint32_t xk[TPL], xq[TPL];
        float2 xl[TPL];
        struct ScanSrc {
            __amdgpu_buffer_rsrc_t k, q, l;
        };
        // chunk sources advance by one chunk of rows per step (no 64-bit
        // multiplies in the loop)
        const size_t step_el = (size_t)CH * rowel;
        size_t src_el = ((size_t)t0 * H + h) * DK;   // first element of the next chunk to load
        int64_t src_rem = t1 - t0;                     // its rows left in the sequence
        auto scan_src = [&]() {
            const int nv = src_rem <= 0 ? 0 : (src_rem < CH ? (int)src_rem : CH);
            const ScanSrc r{make_rsrc((const __bf16*)p.k + src_el, span_bytes(nv, 2)),
                            make_rsrc((const __bf16*)p.q + src_el, span_bytes(nv, 2)),
                            make_rsrc(p.la + src_el, span_bytes(nv, 4))};
            src_el += step_el;
            src_rem -= CH;
            return r;
        };
        auto load_kq = [&](const ScanSrc& r, int tau) {
            const int el = (part * TPL + tau) * rowel + sc;
            xk[tau] = __builtin_amdgcn_raw_buffer_load_b32(r.k, el * 2, 0, 0);
            if constexpr (WANT_O) xq[tau] = __builtin_amdgcn_raw_buffer_load_b32(r.q, el * 2, 0, 0);
        };
        auto load_la = [&](const ScanSrc& r, int tau) {
            const int el = (part * TPL + tau) * rowel + sc;
            auto lv = __builtin_amdgcn_raw_buffer_load_b64(r.l, el * 4, 0, 0);
            xl[tau] = make_float2(__uint_as_float(lv[0]), __uint_as_float(lv[1]));
        };
        // Exclusive prefix `pre` over the four parts, the decay `e0` of parts
        // 0 and 1 and the chunk total `tot`, each formed in one fixed order.
        auto scan4 = [&](float a, float& pre, float& e0, float& tot) {
            const bool odd = part & 1, upper = part & 2;
            const float b = lane_xor16(a);
            const float lo = odd ? b : a, hi = odd ? a : b;
            const float ps = lo + hi;
            const float c = lane_xor32(ps);
            const float plo = upper ? c : ps, phi = upper ? ps : c;
            tot = plo + phi;
            e0 = plo;
            pre = (upper ? plo : 0.f) + (odd ? lo : 0.f);
        };
        {
            const ScanSrc r = scan_src();
#pragma unroll
            for (int tau = 0; tau < TPL; ++tau) {
                load_kq(r, tau);
                load_la(r, tau);
            }
        }
        int b3 = 0;   // chunk c % 3
        for (int64_t c = 0; c < nch + 2; ++c) {   // step c - 2 scans chunk c
            if (c < nch) {
                const int b2 = (int)(c & 1);
                const ScanSrc nx = scan_src();
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
                float pre0, pre1, E00, E01, tot0, tot1;
                scan4(a0, pre0, E00, tot0);
                scan4(a1, pre1, E01, tot1);
                const float ee0 = __builtin_amdgcn_exp2f(E00), ee1 = __builtin_amdgcn_exp2f(E01);
                if (part == 0) {
                    *reinterpret_cast<float2*>(&sVec[b3][0][sc]) = make_float2(ee0, ee1);
                    *reinterpret_cast<float2*>(&sVec[b3][1][sc]) =
                        make_float2(__builtin_amdgcn_exp2f(tot0 - E00), __builtin_amdgcn_exp2f(tot1 - E01));
                }
                const float o0 = pre0 - E00, o1 = pre1 - E01;
                // LDS byte addresses of this lane's first row; rows follow at
                // constant strides, which the stores take as immediate offsets
                const int e0 = part * TPL * LDR + sc;
                const uint32_t aX = lds_addr(sX[b3] + e0), aQ = lds_addr(sQX[b2] + e0),
                               aQl = lds_addr(sQXl[b2] + e0), aY = lds_addr(sY[b3] + e0),
                               aYl = lds_addr(sYl[b3] + e0), aQp = lds_addr((const __bf16*)(sQp[b3] + e0));
                auto st = [](uint32_t a, uint32_t v) {
                    *(__attribute__((address_space(3))) uint32_t*)(uintptr_t)a = v;
                };
#pragma unroll
                for (int tau = 0; tau < TPL; ++tau) {
                    const float d0 = cs0[tau] + o0, d1 = cs1[tau] + o1;
                    const float fx0 = __builtin_amdgcn_exp2f(d0), fx1 = __builtin_amdgcn_exp2f(d1);
                    const float fy0 = __builtin_amdgcn_exp2f(-d0), fy1 = __builtin_amdgcn_exp2f(-d1);
                    if constexpr (WANT_O) {
                        const float2 kf = bf2_to_f2(xk[tau]), qf = bf2_to_f2(xq[tau]);
                        load_kq(nx, tau);
                        const float X0 = kf.x * fx0, X1 = kf.y * fx1;
                        const float Q0 = qf.x * fx0, Q1 = qf.y * fx1;
                        const float Y0 = kf.x * fy0, Y1 = kf.y * fy1;
                        const uint32_t qh = f2_to_bf2(Q0, Q1);
                        const uint32_t yh = f2_to_bf2(Y0, Y1);
                        const float2 qhf = bf2_to_f2(qh), yhf = bf2_to_f2(yh);
                        const uint32_t ro = tau * LDR * 2;
                        st(aX + ro, f2_to_bf2(X0, X1));
                        st(aQ + ro, qh);
                        st(aQl + ro, f2_to_bf2(Q0 - qhf.x, Q1 - qhf.y));
                        st(aY + ro, yh);
                        st(aYl + ro, f2_to_bf2(Y0 - yhf.x, Y1 - yhf.y));
                        // q e^{g} = QX e^{E0} in fp16 (at most |q|)
                        st(aQp + ro, pack_h2(Q0 * ee0, Q1 * ee1));
                    } else {
                        // k only: X, Y (hi, lo)
                        const float2 kf = bf2_to_f2(xk[tau]);
                        load_kq(nx, tau);
                        const float X0 = kf.x * fx0, X1 = kf.y * fx1;
                        const float Y0 = kf.x * fy0, Y1 = kf.y * fy1;
                        const uint32_t yh = f2_to_bf2(Y0, Y1);
                        const float2 yhf = bf2_to_f2(yh);
                        const uint32_t ro = tau * LDR * 2;
                        st(aX + ro, f2_to_bf2(X0, X1));
                        st(aY + ro, yh);
                        st(aYl + ro, f2_to_bf2(Y0 - yhf.x, Y1 - yhf.y));
                    }
                }
                b3 = b3 == 2 ? 0 : b3 + 1;
            }
            __syncthreads();
        }
    } else {
        // ==================================================== tile waves
        float pbp[2][4], pbn[2][4];   // beta of the chunk being tiled / the next one
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) pbp[tb][r] = 0.f;
        for (int64_t s = -2; s < nch; ++s) {
            const int64_t c = s + 1;
            load_beta(c + 1, pbn);
            if (c >= 0 && c < nch) {
                const int b3 = (int)(c % 3), b2 = (int)(c & 1);
                const __bf16* X = sX[b3];
                const __bf16* QX = sQX[b2];
                const __bf16* Yh = sY[b3];
                const __bf16* Yl = sYl[b3];
                const __bf16* QXl = sQXl[b2];
                float* Tb = sT[b2];
                __bf16* Mh = sMh[b2];
                __bf16* Ml = sMl[b2];
                if (role == 0) {
                    const f32x4 l00 = block(X, X, 0, Yh, Yh, 0, false);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = g * 4 + r;
                        Tb[row * LDM + ln] = ln < row ? pbp[0][r] * l00[r] : 0.f;
                    }
                    wave_lds_sync();
                    invert16(Tb, Tb, lane);   // in place: all reads precede the writes
                } else if (role == 1) {
                    const f32x4 l11 = block(X, X, 16, Yh, Yh, 16, false);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = g * 4 + r;
                        Tb[(16 + row) * LDM + 16 + ln] = ln < row ? pbp[1][r] * l11[r] : 0.f;
                    }
                    wave_lds_sync();
                    invert16(Tb + 16 * LDM + 16, Tb + 16 * LDM + 16, lane);
                } else if (role == 2) {
                    // -L10 (beta-scaled) goes where the consumers read it
                    const f32x4 v = block(X, X, 16, Yh, Yh, 0, false);
#pragma unroll
                    for (int r = 0; r < 4; ++r) Tb[(16 + g * 4 + r) * LDM + ln] = -pbp[1][r] * v[r];
                    if constexpr (WANT_O) store_m(Mh, Ml, block(QX, QXl, 0, Yh, Yl, 0, true), 0, 0, true);
                } else if constexpr (WANT_O) {
                    f32x4 m10, m11;
                    block2(QX, QXl, 16, Yh, Yl, 0, 16, m10, m11);
                    store_m(Mh, Ml, m10, 16, 0, false);
                    store_m(Mh, Ml, m11, 16, 16, true);
                }
            }
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int r = 0; r < 4; ++r) pbp[tb][r] = pbn[tb][r];
            __syncthreads();
        }
    }
}

hipError_t launch_chunk_fwd_pipe(const PrefillParams& p, hipStream_t stream) {
    const int64_t groups = ((int64_t)p.n_units + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * p.n_slices)), block(64 * (8 + KDA_PIPE_NSCAN));
    // the per-chunk outputs are only kept for the backward pass, which takes
    // no o (the launch is refused if both are asked for)
    if (p.h_states && p.o) return hipErrorInvalidValue;
    // segments of two lengths: equal-length sequences writing o, no window
    const bool seg = p.seg_r0 != 0 || (p.seg_first != 0 && p.seg_first != p.seg_len);
    if (seg && (p.cu || p.seg_sel >= 0 || !p.o || p.seg_first <= 0)) return hipErrorInvalidValue;
    if (seg)
        hipLaunchKernelGGL((chunk_fwd_pipe_kernel<KDA_PIPE_NSCAN, false, true, true>), grid, block, 0, stream, p);
    else if (p.h_states)
        hipLaunchKernelGGL((chunk_fwd_pipe_kernel<KDA_PIPE_NSCAN, true, false, false>), grid, block, 0, stream, p);
    else if (p.o)
        hipLaunchKernelGGL((chunk_fwd_pipe_kernel<KDA_PIPE_NSCAN, false, true, false>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((chunk_fwd_pipe_kernel<KDA_PIPE_NSCAN, false, false, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda
