// Measurement probes (built into their own library, libkda_probe.so, never
// into libkda.so): the contraction-phase probe below, and a plain in-place
// stream over a large fp32 buffer (the decode step's access pattern without
// its arithmetic), which measures the HBM bandwidth a read-then-write pass
// reaches on the device.
//
// Contraction-phase probe.
//
// The pipelined prefill's consumer waves spend each 32-token chunk in two
// matrix-core phases: K+ S / Q+ S (per k-slice: the state tile packed to fp16
// for Q+ S, scaled by e^{E0} and packed to bf16 for K+ S, then one bf16 and
// one fp16 16x16x32 product per 16-token row block) and the state update
// S <- e^{E1-E0} (S~ + Y^T U) (per 16-key tile: two transposing LDS reads
// and three bf16 16x16x32 products, then the scaling).  This kernel runs
// exactly those instruction sequences on operands already staged in LDS,
// one wave per SIMD and nothing else on the compute unit, so that rocprof's
// matrix-core counters measure what the phases reach when they are not
// sharing their SIMD with the decay scan and the tile waves (the isolation
// of the contraction phases the operator's target is stated for).
//
//   mode 0: K+ S / Q+ S only;  mode 1: state update only;  mode 2: both.
//
// The LDS operands are filled once from a fixed integer hash (no input
// data), and every result is carried across iterations and written out at
// the end, so no product can be dropped by the compiler.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_chunk.h"

namespace kda {
namespace {

constexpr int PLDR = DK + 8;   // token-major row stride, as in the prefill
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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
__device__ __forceinline__ f16x8 load_tile_h(const uint16_t* p) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    const uint2 b = *reinterpret_cast<const uint2*>(p + 16);
    const uint4 v = make_uint4(a.x, a.y, b.x, b.y);
    return __builtin_bit_cast(f16x8, v);
}
__device__ __forceinline__ bf16x8 load_tr(uint32_t a, int key0) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef short v8s __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(uintptr_t)(a + 2 * key0));
    const v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(uintptr_t)(a + 2 * (key0 + 16 * PLDR)));
    const v8s c = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return __builtin_bit_cast(bf16x8, c);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
// small deterministic values in about [-0.5, 0.5)
__device__ __forceinline__ float hval(uint32_t i) {
    i ^= i >> 16;
    i *= 0x7feb352du;
    i ^= i >> 15;
    i *= 0x846ca68bu;
    i ^= i >> 16;
    return (float)(i & 0xffff) * (1.f / 65536.f) - 0.5f;
}

}  // namespace

__global__ __launch_bounds__(256) void contraction_probe_kernel(float* out, int iters, int mode) {
    typedef Frag<false> Fr;
    __shared__ __attribute__((aligned(16))) __bf16 sX[CH * PLDR];
    __shared__ __attribute__((aligned(16))) uint16_t sQp[CH * PLDR];
    __shared__ __attribute__((aligned(16))) __bf16 sY[CH * PLDR];
    __shared__ __attribute__((aligned(16))) __bf16 sYl[CH * PLDR];
    __shared__ __attribute__((aligned(16))) float sVec[2][DK];
    // keeps a second workgroup off the compute unit: one wave per SIMD
    __shared__ float sPad[24 * 1024];
    const int tid = threadIdx.x, lane = tid & 63;
    sPad[tid * 96] = (float)tid;
    const int g = lane >> 4, ln = lane & 15;
    for (int e = tid; e < CH * PLDR; e += 256) {
        sX[e] = (__bf16)hval(3 * e + 1);
        const _Float16 h = (_Float16)hval(5 * e + 2);
        sQp[e] = __builtin_bit_cast(uint16_t, h);
        const float y = hval(7 * e + 3);
        sY[e] = (__bf16)y;
        sYl[e] = (__bf16)(y * (1.f / 256.f));
    }
    if (tid < 2 * DK) (&sVec[0][0])[tid] = 1.f + 0.01f * hval(tid + 11);
    __syncthreads();

    f32x4 S[8];
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[it][r] = hval(blockIdx.x * 4096 + tid * 32 + it * 4 + r);
    f32x4 R[2] = {}, O[2] = {};
    Fr bUh, bUl;
    {
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = hval(tid * 8 + e + 99);
        SplitBF<8> s8 = split8(f);
        bUh.v = s8.hi;
        bUl.v = s8.lo;
    }
    const int aoff = ln * PLDR + g * 4;
    const int troff = (4 * g + (ln >> 2)) * PLDR + 4 * (ln & 3);
    const float* e0 = sVec[0] + g * 4;
    const float* e1 = sVec[1] + g * 4;
    const bool kq = mode != 1, upd = mode != 0;
    for (int i = 0; i < iters; ++i) {
        if (kq) {
            // ---- K+ S / Q+ S, as the consumer waves run it
            const __bf16* Xb = sX + aoff;
            const uint16_t* Qb = sQp + aoff;
            Fr aK[2][2];
            f16x8 aQ[2][2];
            float4 ev[2][2];
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                load_tile(aK[0][tb], Xb + tb * 16 * PLDR);
                aQ[0][tb] = load_tile_h(Qb + tb * 16 * PLDR);
                ev[0][tb] = *reinterpret_cast<const float4*>(e0 + tb * 16);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int cur = ks & 1;
                if (ks < 3) {
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) {
                        load_tile(aK[cur ^ 1][tb], Xb + tb * 16 * PLDR + (ks + 1) * 32);
                        aQ[cur ^ 1][tb] = load_tile_h(Qb + tb * 16 * PLDR + (ks + 1) * 32);
                        ev[cur ^ 1][tb] = *reinterpret_cast<const float4*>(e0 + (2 * ks + 2 + tb) * 16);
                    }
                }
                f16x8 bS16;
                Fr bS;
                {
                    u32x4 w;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        w[2 * j] = pack_h2(S[2 * ks + j][0], S[2 * ks + j][1]);
                        w[2 * j + 1] = pack_h2(S[2 * ks + j][2], S[2 * ks + j][3]);
                    }
                    bS16 = __builtin_bit_cast(f16x8, w);
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float4 sc4 = ev[cur][j];
                        S[2 * ks + j][0] *= sc4.x;
                        S[2 * ks + j][1] *= sc4.y;
                        S[2 * ks + j][2] *= sc4.z;
                        S[2 * ks + j][3] *= sc4.w;
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
                    O[tb] = mfma32h(aQ[cur][tb], bS16, O[tb]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (upd) {
            // ---- S <- e^{E1-E0} (S~ + Y^T U), as the consumer waves run it
            const uint32_t Yb = lds_addr(sY + troff);
            const uint32_t Ylb = lds_addr(sYl + troff);
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
            const float4 a4 = *reinterpret_cast<const float4*>(e1 + 7 * 16);
            S[7][0] *= a4.x;
            S[7][1] *= a4.y;
            S[7][2] *= a4.z;
            S[7][3] *= a4.w;
        }
    }
    float* o = out + ((size_t)blockIdx.x * 256 + tid) * 48;
    o[47] = sPad[((tid + 1) & 255) * 96];
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[it * 4 + r] = S[it][r];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            o[32 + tb * 4 + r] = R[tb][r];
            if (tb * 4 + r < 7) o[40 + tb * 4 + r] = O[tb][r];
        }
}

}  // namespace kda

// Matrix-core flops one launch issues: 16 (K+ S / Q+ S) and 24 (update)
// 16x16x32 products of 16384 flops per wave and iteration.
namespace kda {
namespace {
// x <- a x in place over n4 float4s: every wave instruction moves 1 KB of
// consecutive memory (64 lanes x 16 B), nontemporal loads and stores, 8
// loads in flight per lane before the first store; grid-stride over
// 8 KB-per-wave blocks, and a tail of single float4s.
typedef float v4f __attribute__((ext_vector_type(4)));
// mode 0: x <- a x in place; 1: y <- a x; 2: read x only (one sum per lane
// written to y, so no load can be dropped).
template <int MODE>
__global__ __launch_bounds__(1024) void stream_probe_kernel(v4f* x, v4f* y, int64_t n4, float a) {
    constexpr int U = 8;
    const int64_t lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int64_t n_blk = n4 / (64 * U);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t b = wave; b < n_blk; b += n_waves) {
        const int64_t o = b * (64 * U) + lane;
        v4f v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(x + o + 64 * u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (MODE == 0) __builtin_nontemporal_store(v[u] * a, x + o + 64 * u);
            else if constexpr (MODE == 1) __builtin_nontemporal_store(v[u] * a, y + o + 64 * u);
            else acc += v[u];
        }
    }
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = n_blk * (64 * U) + t; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        if constexpr (MODE == 0) x[i] = x[i] * a;
        else if constexpr (MODE == 1) y[i] = x[i] * a;
        else acc += x[i];
    }
    if constexpr (MODE == 2) y[t] = acc;
}
}  // namespace
}  // namespace kda

// x: n_floats fp32 (a multiple of 4, 16-byte aligned); n_wg workgroups of
// 1024 threads.  mode 0: x <- a x in place (y unused); mode 1: y <- a x
// (y as large as x); mode 2: read x, y receives n_wg * 1024 float4 partial
// sums.  Returns a hipError_t.
extern "C" int kda_probe_stream(float* x, float* y, int64_t n_floats, float a, int n_wg, int mode,
                                hipStream_t stream) {
    if (!x || n_floats < 4 || (n_floats & 3) || ((uintptr_t)x & 15) || n_wg < 1 || mode < 0 ||
        mode > 2 || (mode != 0 && (!y || ((uintptr_t)y & 15))))
        return (int)hipErrorInvalidValue;
    kda::v4f* xv = (kda::v4f*)x;
    kda::v4f* yv = (kda::v4f*)y;
    const int64_t n4 = n_floats / 4;
    if (mode == 0)
        hipLaunchKernelGGL(kda::stream_probe_kernel<0>, dim3(n_wg), dim3(1024), 0, stream, xv, yv, n4, a);
    else if (mode == 1)
        hipLaunchKernelGGL(kda::stream_probe_kernel<1>, dim3(n_wg), dim3(1024), 0, stream, xv, yv, n4, a);
    else
        hipLaunchKernelGGL(kda::stream_probe_kernel<2>, dim3(n_wg), dim3(1024), 0, stream, xv, yv, n4, a);
    return (int)hipGetLastError();
}

extern "C" double kda_probe_flops(int n_wg, int iters, int mode) {
    const double per = (mode != 1 ? 16.0 : 0.0) + (mode != 0 ? 24.0 : 0.0);
    return per * 16384.0 * 4.0 * n_wg * (double)iters;
}

// out: n_wg * 256 * 48 floats.  Returns a hipError_t.
extern "C" int kda_probe_contraction(float* out, int n_wg, int iters, int mode,
                                     hipStream_t stream) {
    if (!out || n_wg < 1 || iters < 1 || mode < 0 || mode > 2) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(kda::contraction_probe_kernel, dim3(n_wg), dim3(256), 0, stream, out, iters,
                       mode);
    return (int)hipGetLastError();
}
