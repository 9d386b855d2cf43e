// Device-side helpers shared by the KDA kernels (gfx950 only).
//
// Matrix-core conventions (CDNA3/CDNA4 16x16 MFMA family, wave64):
//   * A 16x16 fp32 accumulator tile is held as f32x4 per lane: lane l owns
//     column (l & 15) and rows 4*(l >> 4) + r, r = 0..3 ("C layout").
//   * An operand slab of 16 rows x 32 k (bf16 16x16x32) or 16 x 4 k (fp32
//     16x16x4) gives lane l row (l & 15).  Which k a lane supplies only has
//     to agree between the A and the B operand, so every product here picks
//     the k -> (lane group, element) map that lets the B operand be taken
//     straight from C-layout accumulator registers: for a 32-k slab made of
//     two stacked 16-row C tiles, lane group g = l >> 4 supplies
//     k = 4g + e (e = 0..3) from the first tile and 16 + 4g + e from the
//     second ("tile order").  A 16-k slab uses only the first half.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

// Round-to-nearest-even bf16 and the residual lo = bf16(x - hi): hi + lo
// carries 16 significant bits.
template <int N>
struct SplitBF;

template <>
struct SplitBF<8> {
    bf16x8 hi, lo;
};
template <>
struct SplitBF<4> {
    bf16x4 hi, lo;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two floats to a packed bf16 pair (round to nearest even), and back.  The
// empty asm emits nothing; it hides the packed value's origin so that the
// compiler keeps one paired conversion instead of re-deriving each half with
// a conversion of its own when only that half is inspected (which doubles
// the conversions of a hi/lo split).  The conversion itself stays an
// ordinary compiler-generated instruction.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    bf16x2_t r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    uint32_t u = __builtin_bit_cast(uint32_t, r);
    asm("" : "+v"(u));
    return u;
}
__device__ __forceinline__ float bf2_first(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf2_second(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ bf16x8 round8(const float (&x)[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf2(x[2 * i], x[2 * i + 1]);
    return __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ bf16x4 round4(const float (&x)[4]) {
    u32x2 w;
#pragma unroll
    for (int i = 0; i < 2; ++i) w[i] = pack_bf2(x[2 * i], x[2 * i + 1]);
    return __builtin_bit_cast(bf16x4, w);
}
// Pairwise: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ SplitBF<8> split8(const float (&x)[8]) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pack_bf2(x[2 * i], x[2 * i + 1]);
        l[i] = pack_bf2(x[2 * i] - bf2_first(h[i]), x[2 * i + 1] - bf2_second(h[i]));
    }
    SplitBF<8> s;
    s.hi = __builtin_bit_cast(bf16x8, h);
    s.lo = __builtin_bit_cast(bf16x8, l);
    return s;
}
__device__ __forceinline__ SplitBF<4> split4(const float (&x)[4]) {
    u32x2 h, l;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        h[i] = pack_bf2(x[2 * i], x[2 * i + 1]);
        l[i] = pack_bf2(x[2 * i] - bf2_first(h[i]), x[2 * i + 1] - bf2_second(h[i]));
    }
    SplitBF<4> s;
    s.hi = __builtin_bit_cast(bf16x4, h);
    s.lo = __builtin_bit_cast(bf16x4, l);
    return s;
}

// Precision of one product:
//   PLAIN : both operands rounded to bf16 once (1 MFMA)
//   SPLITB: A rounded once, B split hi+lo (2 MFMAs)
//   SPLIT2: both split, lo*lo dropped (3 MFMAs)
// With F32 = true every mode is one exact-fp32 pass on 16x16x4 fp32 MFMA.
enum Mode { PLAIN = 1, SPLITB = 2, SPLIT2 = 3 };

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma4f(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += A(16 x 32) * B(32 x 16), one lane's 8 k-values of each operand.
template <bool F32, int MODE>
__device__ __forceinline__ void mma_k32(f32x4& acc, const float (&a)[8], const float (&b)[8]) {
    if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = mfma4f(a[e], b[e], acc);
    } else if constexpr (MODE == PLAIN) {
        acc = mfma32(round8(a), round8(b), acc);
    } else if constexpr (MODE == SPLITB) {
        bf16x8 ah = round8(a);
        SplitBF<8> bs = split8(b);
        acc = mfma32(ah, bs.lo, acc);
        acc = mfma32(ah, bs.hi, acc);
    } else {
        SplitBF<8> as = split8(a), bs = split8(b);
        acc = mfma32(as.lo, bs.hi, acc);
        acc = mfma32(as.hi, bs.lo, acc);
        acc = mfma32(as.hi, bs.hi, acc);
    }
}

// Same with pre-split operands (when one fragment feeds several products).
struct Frag8 {
    float f[8];        // fp32 values (used by the F32 path)
    bf16x8 hi, lo;     // bf16 split (bf16 path)
};

template <bool F32, int MODE>
__device__ __forceinline__ void prep8(Frag8& fr) {
    if constexpr (!F32) {
        if constexpr (MODE == PLAIN) {
            fr.hi = round8(fr.f);
        } else {
            SplitBF<8> s = split8(fr.f);
            fr.hi = s.hi;
            fr.lo = s.lo;
        }
    }
}

// MODE applies to the pair: PLAIN (a.hi*b.hi), SPLITB (a.hi*(b.hi+b.lo)),
// SPLIT2 (a.hi*b.hi + a.hi*b.lo + a.lo*b.hi).
template <bool F32, int MODE>
__device__ __forceinline__ void mma_k32(f32x4& acc, const Frag8& a, const Frag8& b) {
    if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = mfma4f(a.f[e], b.f[e], acc);
    } else if constexpr (MODE == PLAIN) {
        acc = mfma32(a.hi, b.hi, acc);
    } else if constexpr (MODE == SPLITB) {
        acc = mfma32(a.hi, b.lo, acc);
        acc = mfma32(a.hi, b.hi, acc);
    } else {
        acc = mfma32(a.lo, b.hi, acc);
        acc = mfma32(a.hi, b.lo, acc);
        acc = mfma32(a.hi, b.hi, acc);
    }
}

// acc += A(16 x 16) * B(16 x 16) with lane group g supplying k = 4g + e.
template <bool F32, int MODE>
__device__ __forceinline__ void mma_k16(f32x4& acc, const float (&a)[4], const float (&b)[4]) {
    if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma4f(a[e], b[e], acc);
    } else if constexpr (MODE == PLAIN) {
        acc = mfma16(round4(a), round4(b), acc);
    } else if constexpr (MODE == SPLITB) {
        bf16x4 ah = round4(a);
        SplitBF<4> bs = split4(b);
        acc = mfma16(ah, bs.lo, acc);
        acc = mfma16(ah, bs.hi, acc);
    } else {
        SplitBF<4> as = split4(a), bs = split4(b);
        acc = mfma16(as.lo, bs.hi, acc);
        acc = mfma16(as.hi, bs.lo, acc);
        acc = mfma16(as.hi, bs.hi, acc);
    }
}

// Sum over the 64 lanes of a wave, every lane receiving the total, without
// an LDS round trip: quad butterflies and row rotations by DPP, then the
// gfx950 16- and 32-lane swaps.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over the 32 lanes of each half wave (lanes with equal l >> 5).
__device__ __forceinline__ float half_sum_dpp(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_mov<0x124>(x);   // row_ror:4
    x += dpp_mov<0x128>(x);   // row_ror:8
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x += __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
    return x;
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
    x = half_sum_dpp(x);
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x += __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
    return x;
}
// Value of lane l ^ 32.
__device__ __forceinline__ float swap_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Make LDS writes of this wave visible to all of its lanes and keep the
// compiler from moving LDS accesses across this point (one-wave barrier).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Raw buffer resource over `bytes` bytes from `base`: loads at offsets
// beyond the range return 0, which masks the tokens past a sequence's end
// without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Workgroup barrier that orders LDS only: the fences are limited to the
// local address space, so outstanding global loads and stores stay in
// flight across it (a plain __syncthreads waits for all of them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// The same within one wave.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace kda
