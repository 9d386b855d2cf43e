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
// are HBM-bound.  Prologue: a wave owns one head's 128 channels (two per
// lane) of eight consecutive rows, with the conv weights and the last three
// raw inputs kept in registers, and sums over the row by DPP wave
// reduction.  Epilogue: a lane owns four channels of one of two consecutive
// rows, so every wave instruction moves 1 KB, and a wave reads the inputs
// of four row pairs before it reduces the first (half-wave DPP sums).  The prologue reads and writes through buffer
// resources with 32-bit offsets from its first row (rows past the end read
// as zero, and the window before a sequence start takes the cache entry
// through the same out-of-range trick instead of a branch).  The cache
// update runs as a separate launch after the prologue, so no wave reads a
// cache entry that another already overwrote.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int LY_THREADS = 256;   // 4 rows per workgroup
constexpr float LY_EPS = 1e-6f;

// sigmoid with the hardware reciprocal (about 1 ulp) instead of a correctly
// rounded division
__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

__device__ __forceinline__ float wave_sum(float x) { return wave_sum_dpp(x); }

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

// Packed sequences: the sequence of a token row (largest s with
// cu[s] <= row) and the row's position in it.
__device__ __forceinline__ void locate_packed(int64_t row, const int32_t* cu, int32_t n_seqs,
                                              int64_t& n, int64_t& pos) {
    int lo = 0, hi = n_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)cu[mid] <= row) lo = mid;
        else hi = mid;
    }
    n = lo;
    pos = row - cu[lo];
}

constexpr int LY_TOK = 8;   // consecutive token rows per wave in the prologue (2: 0.55 ms, 4: 0.42, 8: 0.39, 16: 0.88 at T=8192 H=96)

// Two channels of one row through a buffer resource (offsets past its
// range read as zero).
template <typename T>
__device__ __forceinline__ float2 bload2(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ float2 bload2<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x2 u = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    return make_float2(__uint_as_float(u[0]), __uint_as_float(u[1]));
}
template <>
__device__ __forceinline__ float2 bload2<__bf16>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}
__device__ __forceinline__ void bstore2(float2 v, __amdgpu_buffer_rsrc_t r, uint32_t off, float) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, make_float2(v.x, v.y)), r, off, 0, 0);
}
__device__ __forceinline__ void bstore2(float2 v, __amdgpu_buffer_rsrc_t r, uint32_t off, __bf16) {
    __builtin_amdgcn_raw_buffer_store_b32(pack_bf2(v.x, v.y), r, off, 0, 0);
}
constexpr uint32_t OOB = 0x80000000u;   // an offset past every range: reads 0

template <typename InT>
__global__ __launch_bounds__(LY_THREADS) void prologue_kernel(LayerParams p) {
    // workgroup = (block of LY_TOK token rows, group of four heads, one per
    // wave); a wave keeps its head's conv weights and the last three raw
    // inputs in registers while it walks its rows
    constexpr int ES = (int)sizeof(InT);
    const int lane = threadIdx.x & 63;
    const uint32_t nhg = (uint32_t)(p.H + 3) / 4;
    const uint32_t blk = blockIdx.x;
    const uint32_t tb = blk / nhg;
    const int h = (int)(blk - tb * nhg) * (LY_THREADS / 64) +
                  __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (h >= p.H) return;
    const int H = p.H;
    const int c = 2 * lane;
    const int64_t HD = (int64_t)H * 128;
    const int64_t row0 = (int64_t)tb * LY_TOK;
    const int nt = p.rows - row0 < LY_TOK ? (int)(p.rows - row0) : LY_TOK;
    // buffer resources over this head's rows [wb, row0 + nt): offsets count
    // from row wb, channel 0; rows past the end read as zero
    const int64_t wb = row0 >= 3 ? row0 - 3 : 0;
    const int nrow = (int)(row0 + nt - wb);
    const int rb_in = (int)HD * ES, rb_f = (int)HD * 4;   // bytes per token row
    const int64_t e0 = wb * HD + (int64_t)h * 128;
    const int sp_in = (nrow - 1) * rb_in + 128 * ES, sp_f = (nrow - 1) * rb_f + 512;
    __amdgpu_buffer_rsrc_t rin[3], rout[3];
    rin[0] = make_rsrc((const InT*)p.q_raw + e0, sp_in);
    rin[1] = make_rsrc((const InT*)p.k_raw + e0, sp_in);
    rin[2] = make_rsrc((const InT*)p.v_raw + e0, sp_in);
    rout[0] = make_rsrc((InT*)p.q + e0, sp_in);
    rout[1] = make_rsrc((InT*)p.k + e0, sp_in);
    rout[2] = make_rsrc((InT*)p.v + e0, sp_in);
    const auto ra = make_rsrc(p.a + e0, sp_f);
    const auto rla = make_rsrc(p.log_alpha + e0, sp_f);
    const auto rbi = make_rsrc(p.b + wb * H + h, ((nrow - 1) * H + 1) * 4);
    const auto rbo = make_rsrc(p.beta + wb * H + h, ((nrow - 1) * H + 1) * 4);

    // every load first (the stores below may not be reordered above them)
    float4 w[3][2];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        // weights of channels c, c + 1: [tensor, head, channel, tap]
        const float* wp = p.conv_w + (((int64_t)i * H + h) * 128 + c) * 4;
        w[i][0] = *reinterpret_cast<const float4*>(wp);
        w[i][1] = *reinterpret_cast<const float4*>(wp + 4);
    }
    float2 cur[LY_TOK][3], av[LY_TOK];
    float bv[LY_TOK];
#pragma unroll
    for (int tt = 0; tt < LY_TOK; ++tt) {
        const int r = (int)(row0 + tt - wb);   // rows past nt read as zero
#pragma unroll
        for (int i = 0; i < 3; ++i) cur[tt][i] = bload2<InT>(rin[i], r * rb_in + c * ES);
        av[tt] = bload2<float>(ra, r * rb_f + c * 4);
        bv[tt] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbi, r * H * 4, 0, 0));
    }
    // the three inputs before a row: x_{t-3}, x_{t-2}, x_{t-1}, each from
    // the raw rows or, before the sequence start, from the cache (the
    // other source's offset is out of range, so the sum is the one value)
    float2 win[3][3];
    auto fill_window = [&](int64_t row, int64_t n, int64_t pos) {
        const auto rc = make_rsrc(p.cache ? p.cache + n * 9 * HD : nullptr, p.cache ? (int)(9 * HD * 4) : 0);
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int64_t tp = pos - 3 + j;
                const uint32_t o_raw = tp >= 0 ? (uint32_t)((row - 3 + j - wb) * rb_in + c * ES) : OOB;
                // cache tap 3 + tp holds x_{tp}
                const uint32_t o_c = tp < 0 ? (uint32_t)((((i * 3 + 3 + tp) * H + h) * 128 + c) * 4) : OOB;
                const float2 x = bload2<InT>(rin[i], o_raw), y = bload2<float>(rc, o_c);
                win[i][j] = make_float2(x.x + y.x, x.y + y.y);
            }
    };
    // equal lengths: sequence and position of the first row, then counted on
    int64_t n = 0, pos = 0;
    if (!p.cu) {
        n = row0 / p.T;
        pos = row0 - n * p.T - 1;
    }
#pragma unroll
    for (int tt = 0; tt < LY_TOK; ++tt) {
        if (tt >= nt) break;
        const int64_t row = row0 + tt;
        if (p.cu) {
            locate_packed(row, p.cu, p.n_seqs, n, pos);
        } else if (++pos == p.T) {
            ++n;
            pos = 0;
        }
        if (tt == 0 || pos == 0) fill_window(row, n, pos);
        const uint32_t o_in = (uint32_t)((row - wb) * rb_in + c * ES), o_f = (uint32_t)((row - wb) * rb_f + c * 4);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const float2 x3 = cur[tt][i];
            float y0 = w[i][0].x * win[i][0].x;
            float y1 = w[i][1].x * win[i][0].y;
            y0 = fmaf(w[i][0].y, win[i][1].x, y0);
            y1 = fmaf(w[i][1].y, win[i][1].y, y1);
            y0 = fmaf(w[i][0].z, win[i][2].x, y0);
            y1 = fmaf(w[i][1].z, win[i][2].y, y1);
            y0 = fmaf(w[i][0].w, x3.x, y0);
            y1 = fmaf(w[i][1].w, x3.y, y1);
            win[i][0] = win[i][1];
            win[i][1] = win[i][2];
            win[i][2] = x3;
            y0 *= sigm(y0);
            y1 *= sigm(y1);
            if (i < 2) {
                const float r = rsqrtf(wave_sum(y0 * y0 + y1 * y1) + LY_EPS);
                y0 *= r;
                y1 *= r;
            }
            bstore2(make_float2(y0, y1), rout[i], o_in, InT());
        }
        bstore2(make_float2(-5.f * sigm(av[tt].x), -5.f * sigm(av[tt].y)), rla, o_f, 0.f);
        if (lane == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sigm(bv[tt])), rbo,
                                                  (uint32_t)((row - wb) * H * 4), 0, 0);
    }
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
    if (p.cu) {   // clamped into [0, rows]: a malformed table never reads out of bounds
        const int64_t a = p.cu[n], b = p.cu[n + 1];
        start = a < 0 ? 0 : (a > p.rows ? p.rows : a);
        const int64_t e = b < start ? start : (b > p.rows ? p.rows : b);
        L = e - start;
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

// Epilogue: lane l holds channels 4 (l & 31)..+3 of item 2 j + (l >> 5), so a
// wave instruction reads two consecutive items (1 KB); each wave runs
// EP_IT such pairs with every load issued before the first reduction
// (0.183 ms at T=8192 H=96 against 0.213 ms with one item per wave and two
// channels per lane; 8 pairs per wave 0.200 ms).
constexpr int EP_IT = 4;
__global__ __launch_bounds__(LY_THREADS) void epilogue_kernel(const float* __restrict__ o,
                                                              const float* __restrict__ g,
                                                              const float* __restrict__ w,
                                                              float* __restrict__ out, int64_t items) {
    const int lane = threadIdx.x & 63;
    const int64_t first = ((int64_t)blockIdx.x * (LY_THREADS / 64) + (threadIdx.x >> 6)) * (2 * EP_IT);
    const int c = 4 * (lane & 31);
    const float4 ww = *reinterpret_cast<const float4*>(w + c);
    f32x4 x[EP_IT], gg[EP_IT];
#pragma unroll
    for (int j = 0; j < EP_IT; ++j) {
        int64_t item = first + 2 * j + (lane >> 5);
        item = item < items ? item : items - 1;   // a short tail re-reads the last item
        x[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o + item * 128 + c));
        gg[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + item * 128 + c));
    }
#pragma unroll
    for (int j = 0; j < EP_IT; ++j) {
        const int64_t item = first + 2 * j + (lane >> 5);
        const f32x4 v = x[j];
        const float r = rsqrtf(half_sum_dpp(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]) * (1.f / 128.f) + LY_EPS);
        const f32x4 res = {v[0] * r * ww.x * sigm(gg[j][0]), v[1] * r * ww.y * sigm(gg[j][1]),
                           v[2] * r * ww.z * sigm(gg[j][2]), v[3] * r * ww.w * sigm(gg[j][3])};
        if (item < items) __builtin_nontemporal_store(res, reinterpret_cast<f32x4*>(out + item * 128 + c));
    }
}

hipError_t launch_prologue(const LayerParams& p, bool bf16_in, hipStream_t stream) {
    const int64_t items = p.rows * p.H;
    dim3 grid((unsigned)(((p.rows + LY_TOK - 1) / LY_TOK) * ((p.H + 3) / 4))), block(LY_THREADS);
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
        hipLaunchKernelGGL(epilogue_kernel, dim3((unsigned)((items + 8 * EP_IT - 1) / (8 * EP_IT))),
                           dim3(LY_THREADS), 0, stream, o, g, w, out, items);
    return hipGetLastError();
}

}  // namespace kda
