// Helpers shared by the chunkwise prefill kernels (gfx950): tile shapes,
// operand fragment loads, cross-lane scans and the 16 x 16 unit-triangular
// inverse.
#pragma once

#include <type_traits>

#include "kda_device.h"

namespace kda {

constexpr int CH = 32;          // chunk length (tokens)
constexpr int DK = 128;         // key / value head dimension
constexpr int LDM = CH + 4;     // row stride of fp32 [CH][CH] tiles
constexpr float LOG2E = 1.4426950408889634f;

template <bool F32>
struct Tiles {
    typedef typename std::conditional<F32, float, __bf16>::type Op;   // operand element
    static constexpr int LDR = F32 ? DK + 4 : DK + 8;     // token-major row stride
    static constexpr int LDY = F32 ? CH + 4 : CH + 8;     // channel-major row stride
};

// 8 operand values for one lane from a row of operand-type LDS data.
// contiguous: p[0..7];  tile order: p[0..3] and p[16..19].
template <bool F32>
struct Frag {
    typename std::conditional<F32, float[8], bf16x8>::type v;
};

__device__ __forceinline__ void load_contig(Frag<false>& f, const __bf16* p) {
    f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load_tile(Frag<false>& f, const __bf16* p) {
    bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void load_contig(Frag<true>& f, const float* p) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void load_tile(Frag<true>& f, const float* p) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 16);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// acc += A * B for one 16 x 16 x 32 slab.
__device__ __forceinline__ void mma(f32x4& acc, const Frag<false>& a, const Frag<false>& b) {
    acc = mfma32(a.v, b.v, acc);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<true>& a, const Frag<true>& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = mfma4f(a.v[e], b.v[e], acc);
}

template <typename InT>
__device__ __forceinline__ float in_f32(InT x) {
    return to_f32(x);
}


__device__ __forceinline__ float2 bf2_to_f2(uint32_t u) {
    return make_float2(bf2_first(u), bf2_second(u));
}
__device__ __forceinline__ uint32_t f2_to_bf2(float a, float b) { return pack_bf2(a, b); }

// Pack the low (sel = 0x05040100) or high (0x07060302) bf16 halves of two
// dwords into one dword: result = {b.half, a.half}.
__device__ __forceinline__ uint32_t perm2(uint32_t a, uint32_t b, uint32_t sel) {
    return __builtin_amdgcn_perm(a, b, sel);
}
constexpr uint32_t LO_HALVES = 0x05040100u, HI_HALVES = 0x07060302u;

// Broadcast lane qc of every quad (4 consecutive lanes) to the whole quad.
__device__ __forceinline__ float quad_bcast(float x, int qc) {
    const int v = __float_as_int(x);
    switch (qc) {
        case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x00, 0xf, 0xf, false));
        case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x55, 0xf, 0xf, false));
        case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xaa, 0xf, 0xf, false));
        default: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xff, 0xf, 0xf, false));
    }
}

// Value of lane l ^ 32, and of lane l ^ 16 (one cross-row swap each, no
// LDS round trip).
__device__ __forceinline__ float lane_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float lane_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}

// Exclusive prefix `pre` and total `tot` of the per-lane sums `a` over the
// PARTS lanes l, l + 64/PARTS, ... that hold consecutive token runs of one
// channel.  The total is formed in one fixed order, so every part gets the
// same bits.
template <int PARTS>
__device__ __forceinline__ void parts_scan(float a, int part, float& pre, float& tot) {
    if constexpr (PARTS == 2) {
        const float b = lane_xor32(a);
        pre = part ? b : 0.f;
        tot = part ? b + a : a + b;
    } else {
        static_assert(PARTS == 4, "two or four parts");
        const bool odd = part & 1, upper = part & 2;
        const float b = lane_xor16(a);
        const float lo = odd ? b : a, hi = odd ? a : b;
        const float ps = lo + hi;   // sum of the pair of parts
        const float c = lane_xor32(ps);
        const float plo = upper ? c : ps, phi = upper ? ps : c;
        tot = plo + phi;
        pre = (upper ? plo : 0.f) + (odd ? lo : 0.f);
    }
}

// (I + L)^{-1} of a 16 x 16 strictly lower-triangular L (LDS, row stride
// LDM, upper part stored as zeros) by forward substitution on one wave:
// lane 4j + q owns rows q, q+4, q+8, q+12 of column j; at step c the owner
// of x_c broadcasts it to its quad with a DPP quad permute.  The result is
// written to T (same layout).
__device__ __forceinline__ void invert16(const float* L, float* T, int lane) {
    const int j = lane >> 2, q = lane & 3;
    float Lr[4][16];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int c4 = 0; c4 < 16; c4 += 4) {
            const float4 t4 = *reinterpret_cast<const float4*>(L + (q + 4 * k) * LDM + c4);
            Lr[k][c4] = t4.x; Lr[k][c4 + 1] = t4.y; Lr[k][c4 + 2] = t4.z; Lr[k][c4 + 3] = t4.w;
        }
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (q + 4 * k == j) ? 1.f : 0.f;
#pragma unroll
    for (int c = 0; c < 15; ++c) {
        const float xc = quad_bcast(x[c >> 2], c & 3);
        // L[i][c] is zero for i <= c, so rows at or above c are unchanged.
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] -= Lr[k][c] * xc;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) T[(q + 4 * k) * LDM + j] = x[k];
}

}  // namespace kda
