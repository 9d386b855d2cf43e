// One-token KDA decode step, state updated in place (gfx950).
//
// Per (request, head) the step is the three-step update of "Kimi K3 核心算子
// 拆解" (devpress.csdn.net) section 2.3 -- decay S' = Diag(alpha) S, erase
// beta k (k^T S')^T, write beta k v^T -- followed by the readout
// o = S_t^T q ("Kimi K3 技术报告解读" section 3.2).  The page's proposal for a
// fused three-step kernel (section 9.4, no intermediate state in memory) is
// kept; the state is read from HBM once and written once.
//
// The readout needs no second pass over the updated state:
//   q^T S_t = q^T S' + beta (q . k) (v - x)^T,   x = k^T S',
// so one sweep over S produces both reductions x = k^T S' and y = q^T S'.
//
// Work decomposition: one 1024-thread workgroup (16 waves) per (request,
// head) state of 128 x 128 fp32.  Thread t owns value columns 4*(t & 31)..+3
// and key rows (t >> 5) + 32 r, r = 0..3, so every wave instruction touches
// two adjacent 512-byte rows (1 KB contiguous) and each thread keeps only 4
// float4 of the state in flight (this shape measured fastest on MI355X HBM
// for a read-then-write-in-place stream).  The state is streamed with
// nontemporal loads and stores: it is touched once per step and is far
// larger than the caches.  Reductions over the 128 key rows: lanes l and
// l ^ 32 first, then the 16 waves through LDS in two levels.  The launch is
// HBM bound (about 0.86 flop per byte).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int DEC_THREADS = 1024;   // measured best: 512 threads per state ran 4 % slower, 256 13 %

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <typename InT, int NT>
__global__ __launch_bounds__(NT) void decode_step_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    float* __restrict__ S, float* __restrict__ o) {
    constexpr int NW = NT / 64;    // waves
    constexpr int NG = NT / 32;    // row groups
    constexpr int RPT = 128 / NG;  // rows per thread
    const int tid = threadIdx.x;
    const int c4 = tid & 31;       // float4 column
    const int rg = tid >> 5;       // row group: rows rg + NG r
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const size_t bh = blockIdx.x;

    __shared__ float s_k[128], s_q[128], s_a[128], s_v[128];
    __shared__ float s_red[NW][32][9];   // per wave, per float4 column: x[4], y[4]
    __shared__ float s_xy[2][128];              // reduced x, y per value column

    f32x4v* Sp = reinterpret_cast<f32x4v*>(S + bh * (128 * 128));

    // Issue the state stream first; it dominates the step.
    f32x4v s[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) s[r] = __builtin_nontemporal_load(Sp + (rg + NG * r) * 32 + c4);

    if (tid < 128) {
        s_k[tid] = to_f32(k[bh * 128 + tid]);
    } else if (tid < 256) {
        s_q[tid - 128] = to_f32(q[bh * 128 + tid - 128]);
    } else if (tid < 384) {
        s_a[tid - 256] = expf(log_alpha[bh * 128 + tid - 256]);
    } else if (tid < 512) {
        s_v[tid - 384] = to_f32(v[bh * 128 + tid - 384]);
    }
    const float b = beta[bh];
    __syncthreads();

    // q . k, reduced redundantly by every wave (no extra barrier).
    float qk = s_q[lane] * s_k[lane] + s_q[lane + 64] * s_k[lane + 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) qk += __shfl_xor(qk, off);

    // Decay, then partial x = k^T S' and y = q^T S' over this thread's rows.
    float x[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
    float kr[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int row = rg + NG * r;
        const float a = s_a[row], kk = s_k[row], qq = s_q[row];
        kr[r] = kk;
        s[r] *= a;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            x[c] += kk * s[r][c];
            y[c] += qq * s[r][c];
        }
    }
    // Lanes l and l ^ 32 hold the same columns for adjacent row groups.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        x[c] += __shfl_xor(x[c], 32);
        y[c] += __shfl_xor(y[c], 32);
    }
    if (lane < 32) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s_red[wave][c4][c] = x[c];
            s_red[wave][c4][4 + c] = y[c];
        }
    }
    __syncthreads();
    if (tid < 256) {
        // thread (value slot e = tid >> 5, float4 column c = tid & 31) sums the 16 waves
        const int e = tid >> 5, c = tid & 31;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += s_red[w][c][e];
        s_xy[e >> 2][4 * c + (e & 3)] = acc;
    }
    __syncthreads();
    const float4 xv = *reinterpret_cast<const float4*>(&s_xy[0][4 * c4]);
    const float4 yv = *reinterpret_cast<const float4*>(&s_xy[1][4 * c4]);
    const float4 vv = *reinterpret_cast<const float4*>(&s_v[4 * c4]);

    // u = beta (v - x); S_t = S' + k u^T; o = y + (q . k) u.
    float u[4] = {b * (vv.x - xv.x), b * (vv.y - xv.y), b * (vv.z - xv.z), b * (vv.w - xv.w)};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        f32x4v w = s[r];
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] += kr[r] * u[c];
        __builtin_nontemporal_store(w, Sp + (rg + NG * r) * 32 + c4);
    }
    if (rg == 0) {
        float4 ov;
        ov.x = yv.x + qk * u[0];
        ov.y = yv.y + qk * u[1];
        ov.z = yv.z + qk * u[2];
        ov.w = yv.w + qk * u[3];
        reinterpret_cast<float4*>(o + bh * 128)[c4] = ov;
    }
}

hipError_t launch_decode_step(const void* q, const void* k, const void* v, bool bf16_in,
                              const float* log_alpha, const float* beta, float* S,
                              int64_t n_states, float* o, hipStream_t stream) {
    dim3 grid((unsigned)n_states), block(DEC_THREADS);
    if (bf16_in) {
        hipLaunchKernelGGL((decode_step_kernel<__bf16, DEC_THREADS>), grid, block, 0, stream,
                           (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, log_alpha,
                           beta, S, o);
    } else {
        hipLaunchKernelGGL((decode_step_kernel<float, DEC_THREADS>), grid, block, 0, stream, (const float*)q,
                           (const float*)k, (const float*)v, log_alpha, beta, S, o);
    }
    return hipGetLastError();
}

}  // namespace kda
