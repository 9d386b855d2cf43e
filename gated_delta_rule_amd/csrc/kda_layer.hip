// The steps on either side of the KDA recurrence in a layer (gfx950).
//
// Prologue, per token t, head h, channel c ("Kimi K3 四个核心模块的公式与真实
// 张量流" section 1.2; "Kimi K3 核心算子拆解" section 2.6; "Kimi K3 技术报告解读"
// section 3.3):
//   y = sum_{j<4} w[j] x_{t-3+j}   causal depthwise convolution of width 4,
//                                  x_{t<0} from the conv cache (or zeros)
//   q = l2norm(silu(y_q)),  k = l2norm(silu(y_k)),  v = silu(y_v)
//   log_alpha = -5 sigmoid(a),  beta = sigmoid(b)
// with l2norm over the head's 128 channels (eps 1e-6) and the cache holding
// each sequence's last three raw inputs afterwards.
// Epilogue ("把注意力换成一块「会遗忘的内存」" section "层的实现"; gentlecold
// section 1.4): out = o / sqrt(mean o^2 + 1e-6) * w * sigmoid(g).
//
// All three kernels move each element once and do a few flops on it, so they
// are HBM-bound: one wave per (token, head) row of 128 channels (two per
// lane, 8-byte accesses), sums over the row by wave reduction; the previous
// three tokens of the convolution come from the same rows that neighbouring
// waves load, so they are served from cache.  The cache update runs as a
// separate launch after the prologue, so no wave reads a cache entry that
// another already overwrote.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int LY_THREADS = 256;   // 4 rows per workgroup
constexpr float LY_EPS = 1e-6f;

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + __expf(-x)); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <typename T>
__device__ __forceinline__ float2 load2(const T* p);
template <>
__device__ __forceinline__ float2 load2<float>(const float* p) {
    return *reinterpret_cast<const float2*>(p);
}
template <>
__device__ __forceinline__ float2 load2<__bf16>(const __bf16* p) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}
__device__ __forceinline__ void store2(float* p, float2 v) { *reinterpret_cast<float2*>(p) = v; }
__device__ __forceinline__ void store2(__bf16* p, float2 v) {
    bf16x2_t r;
    r[0] = (__bf16)v.x;
    r[1] = (__bf16)v.y;
    *reinterpret_cast<bf16x2_t*>(p) = r;
}

// Sequence of a token row and its position in that sequence.
__device__ __forceinline__ void locate(int64_t row, const int32_t* cu, int32_t n_seqs, int64_t T,
                                       int64_t& n, int64_t& pos) {
    if (!cu) {
        n = row / T;
        pos = row - n * T;
        return;
    }
    int lo = 0, hi = n_seqs;   // largest s with cu[s] <= row
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)cu[mid] <= row) lo = mid;
        else hi = mid;
    }
    n = lo;
    pos = row - cu[lo];
}

template <typename InT>
__global__ __launch_bounds__(LY_THREADS) void prologue_kernel(LayerParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * (LY_THREADS / 64) + (threadIdx.x >> 6);
    if (item >= p.rows * p.H) return;
    const int64_t row = item / p.H;
    const int h = (int)(item - row * p.H);
    int64_t n, pos;
    locate(row, p.cu, p.n_seqs, p.T, n, pos);
    const int c = 2 * lane;
    const int64_t HD = (int64_t)p.H * 128;
    const int64_t base = row * HD + (int64_t)h * 128 + c;

    const InT* raw[3] = {(const InT*)p.q_raw, (const InT*)p.k_raw, (const InT*)p.v_raw};
    InT* out[3] = {(InT*)p.q, (InT*)p.k, (InT*)p.v};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        // weights of channels c, c + 1: [tensor, head, channel, tap]
        const float* wp = p.conv_w + (((int64_t)i * p.H + h) * 128 + c) * 4;
        const float4 w0 = *reinterpret_cast<const float4*>(wp);
        const float4 w1 = *reinterpret_cast<const float4*>(wp + 4);
        const float wa[4] = {w0.x, w0.y, w0.z, w0.w}, wb[4] = {w1.x, w1.y, w1.z, w1.w};
        float y0 = 0.f, y1 = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t tp = pos - 3 + j;   // token x_{t-3+j} of this sequence
            float2 x = make_float2(0.f, 0.f);
            if (tp >= 0) {
                x = load2(raw[i] + base + (tp - pos) * HD);
            } else if (p.cache) {   // cache tap 3 + tp holds x_{tp}
                x = load2(p.cache + (((n * 3 + i) * 3 + (3 + tp)) * p.H + h) * 128 + c);
            }
            y0 = fmaf(wa[j], x.x, y0);
            y1 = fmaf(wb[j], x.y, y1);
        }
        y0 *= sigm(y0);
        y1 *= sigm(y1);
        if (i < 2) {
            const float r = rsqrtf(wave_sum(y0 * y0 + y1 * y1) + LY_EPS);
            y0 *= r;
            y1 *= r;
        }
        store2(out[i] + base, make_float2(y0, y1));
    }
    const float2 a = load2(p.a + base);
    store2(p.log_alpha + base, make_float2(-5.f * sigm(a.x), -5.f * sigm(a.y)));
    if (lane == 0) p.beta[row * p.H + h] = sigm(p.b[row * p.H + h]);
}

// New conv cache: taps m = 0..2 hold x_{L-3+m} of each sequence (length L),
// from the raw inputs or, for short sequences, from the old cache.
template <typename InT>
__global__ __launch_bounds__(LY_THREADS) void conv_cache_kernel(LayerParams p) {
    const int64_t idx = (int64_t)blockIdx.x * LY_THREADS + threadIdx.x;
    const int64_t HD = (int64_t)p.H * 128;
    if (idx >= (int64_t)p.n_seqs * 3 * HD) return;
    const int64_t n = idx / (3 * HD);
    const int64_t rem = idx - n * 3 * HD;
    const int i = (int)(rem / HD);
    const int64_t ch = rem - (int64_t)i * HD;   // h * 128 + c
    int64_t start, L;
    if (p.cu) {
        start = p.cu[n];
        L = p.cu[n + 1] - start;
    } else {
        start = n * p.T;
        L = p.T;
    }
    const InT* raw = i == 0 ? (const InT*)p.q_raw : i == 1 ? (const InT*)p.k_raw : (const InT*)p.v_raw;
    float* cp = p.cache + ((n * 3 + i) * 3) * HD + ch;
    float nv[3];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int64_t tp = L - 3 + m;
        nv[m] = tp >= 0 ? to_f32(raw[(start + tp) * HD + ch]) : cp[(3 + tp) * HD];
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) cp[m * HD] = nv[m];
}

__global__ __launch_bounds__(LY_THREADS) void epilogue_kernel(const float* __restrict__ o,
                                                              const float* __restrict__ g,
                                                              const float* __restrict__ w,
                                                              float* __restrict__ out, int64_t items) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * (LY_THREADS / 64) + (threadIdx.x >> 6);
    if (item >= items) return;
    const int64_t base = item * 128 + 2 * lane;
    const float2 x = *reinterpret_cast<const float2*>(o + base);
    const float2 gg = *reinterpret_cast<const float2*>(g + base);
    const float2 ww = *reinterpret_cast<const float2*>(w + 2 * lane);
    const float r = rsqrtf(wave_sum(x.x * x.x + x.y * x.y) * (1.f / 128.f) + LY_EPS);
    *reinterpret_cast<float2*>(out + base) =
        make_float2(x.x * r * ww.x * sigm(gg.x), x.y * r * ww.y * sigm(gg.y));
}

hipError_t launch_prologue(const LayerParams& p, bool bf16_in, hipStream_t stream) {
    const int64_t items = p.rows * p.H;
    dim3 grid((unsigned)((items + 3) / 4)), block(LY_THREADS);
    if (items > 0) {
        if (bf16_in) hipLaunchKernelGGL(prologue_kernel<__bf16>, grid, block, 0, stream, p);
        else hipLaunchKernelGGL(prologue_kernel<float>, grid, block, 0, stream, p);
    }
    if (p.cache && p.n_seqs > 0) {
        const int64_t n = (int64_t)p.n_seqs * 3 * p.H * 128;
        dim3 g2((unsigned)((n + LY_THREADS - 1) / LY_THREADS));
        if (bf16_in) hipLaunchKernelGGL(conv_cache_kernel<__bf16>, g2, block, 0, stream, p);
        else hipLaunchKernelGGL(conv_cache_kernel<float>, g2, block, 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_epilogue(const float* o, const float* g, const float* w, float* out, int64_t items,
                           hipStream_t stream) {
    if (items > 0)
        hipLaunchKernelGGL(epilogue_kernel, dim3((unsigned)((items + 3) / 4)), dim3(LY_THREADS), 0,
                           stream, o, g, w, out, items);
    return hipGetLastError();
}

}  // namespace kda
