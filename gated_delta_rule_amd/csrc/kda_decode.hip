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
// Work decomposition: one 256-thread workgroup per (request, head) state of
// 128 x 128 fp32 (64 KB).  Thread t owns value columns 4*(t & 31) .. +3 and
// key rows 8 r + (t >> 5), r = 0..15, so each wave's 16 float4 loads cover
// two adjacent 512-byte rows (1 KB contiguous) per instruction.  Reductions
// over the 128 key rows: within a wave by a lane exchange (rows differ in
// t >> 5 parity), across the four waves through LDS.  The launch is HBM
// bound (about 0.86 flop per byte).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int DEC_THREADS = 256;

template <typename InT>
__global__ __launch_bounds__(DEC_THREADS) void decode_step_kernel(
    const InT* __restrict__ q, const InT* __restrict__ k, const InT* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    float* __restrict__ S, float* __restrict__ o) {
    const int tid = threadIdx.x;
    const int cg = tid & 31;       // column group: columns 4cg .. 4cg+3
    const int rg = tid >> 5;       // row group: rows 8r + rg
    const int wave = tid >> 6;
    const size_t bh = blockIdx.x;

    __shared__ float s_k[128], s_q[128], s_a[128], s_v[128];
    __shared__ float s_red[4][32][9];  // per wave: x[4], y[4] per column group

    float4* Sp = reinterpret_cast<float4*>(S + bh * (128 * 128));

    // Issue the state stream first; it dominates the step.
    float4 s[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = Sp[(8 * r + rg) * 32 + cg];

    if (tid < 128) {
        s_k[tid] = to_f32(k[bh * 128 + tid]);
        s_q[tid] = to_f32(q[bh * 128 + tid]);
        s_a[tid] = expf(log_alpha[bh * 128 + tid]);
    } else {
        s_v[tid - 128] = to_f32(v[bh * 128 + tid - 128]);
    }
    const float b = beta[bh];
    __syncthreads();

    // q . k, reduced redundantly by every wave (no extra barrier).
    const int lane = tid & 63;
    float qk = s_q[lane] * s_k[lane] + s_q[lane + 64] * s_k[lane + 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) qk += __shfl_xor(qk, off);

    // Decay, then partial x = k^T S' and y = q^T S' over this thread's rows.
    float x[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
    float kr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * r + rg;
        const float a = s_a[row], kk = s_k[row], qq = s_q[row];
        kr[r] = kk;
        s[r].x *= a;
        s[r].y *= a;
        s[r].z *= a;
        s[r].w *= a;
        x[0] += kk * s[r].x;
        x[1] += kk * s[r].y;
        x[2] += kk * s[r].z;
        x[3] += kk * s[r].w;
        y[0] += qq * s[r].x;
        y[1] += qq * s[r].y;
        y[2] += qq * s[r].z;
        y[3] += qq * s[r].w;
    }
    // Lanes l and l ^ 32 hold the same columns for row groups 2w and 2w+1.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        x[c] += __shfl_xor(x[c], 32);
        y[c] += __shfl_xor(y[c], 32);
    }
    if ((tid & 32) == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            s_red[wave][cg][c] = x[c];
            s_red[wave][cg][4 + c] = y[c];
        }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        x[c] = (s_red[0][cg][c] + s_red[1][cg][c]) + (s_red[2][cg][c] + s_red[3][cg][c]);
        y[c] = (s_red[0][cg][4 + c] + s_red[1][cg][4 + c]) +
               (s_red[2][cg][4 + c] + s_red[3][cg][4 + c]);
    }

    // u = beta (v - x); S_t = S' + k u^T; o = y + (q . k) u.
    float u[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = b * (s_v[4 * cg + c] - x[c]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float4 w = s[r];
        w.x += kr[r] * u[0];
        w.y += kr[r] * u[1];
        w.z += kr[r] * u[2];
        w.w += kr[r] * u[3];
        Sp[(8 * r + rg) * 32 + cg] = w;
    }
    if (rg == 0) {
        float4 ov;
        ov.x = y[0] + qk * u[0];
        ov.y = y[1] + qk * u[1];
        ov.z = y[2] + qk * u[2];
        ov.w = y[3] + qk * u[3];
        reinterpret_cast<float4*>(o + bh * 128)[cg] = ov;
    }
}

hipError_t launch_decode_step(const void* q, const void* k, const void* v, bool bf16_in,
                              const float* log_alpha, const float* beta, float* S,
                              int64_t n_states, float* o, hipStream_t stream) {
    dim3 grid((unsigned)n_states), block(DEC_THREADS);
    if (bf16_in) {
        hipLaunchKernelGGL(decode_step_kernel<__bf16>, grid, block, 0, stream,
                           (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, log_alpha,
                           beta, S, o);
    } else {
        hipLaunchKernelGGL(decode_step_kernel<float>, grid, block, 0, stream, (const float*)q,
                           (const float*)k, (const float*)v, log_alpha, beta, S, o);
    }
    return hipGetLastError();
}

}  // namespace kda
