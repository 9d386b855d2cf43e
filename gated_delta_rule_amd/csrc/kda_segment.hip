// Merge step of the sequence-parallel prefill (gfx950).
//
// A long sequence is cut into segments that run as independent chains.
// Because the recurrence is linear in the state, a segment's final state is
// S_out = F S_in + Sl, where Sl is the segment's final state from a zero
// start and F (d_k x d_k) is the segment's transition, obtained by running
// the same chain from the identity with v = 0.  "Kimi K3 技术报告解读"
// section 7.3 describes this within-GPU sequence parallelism (a segment's
// transition does not depend on its incoming state, so segments run
// independently and merge exactly) next to its multi-GPU form.  The first
// segment starts from the known initial state, so it runs once, directly;
// its final state E opens one left-to-right pass over the middle segments,
//   S_in[0] = E,  S_in[j + 1] = F[j] S_in[j] + Sl[j],
// which gives the incoming state of every later segment (the middle ones
// and the last one, which has no transition of its own), after which those
// segments rerun from their true S_in.
//
// One workgroup per (sequence, head, 16-column block of S): the 128 x 16
// slice of the running state stays in registers, F[j] (64 KB) is staged in
// LDS, and each thread forms 8 outputs as 128-term fp32 dot products in a
// fixed order (deterministic).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int MG_THREADS = 256;
constexpr int MG_COLS = 16;     // value columns per workgroup
constexpr int MG_LDF = 132;     // LDS row stride of F (floats)

__global__ __launch_bounds__(MG_THREADS) void segment_merge_kernel(
    const float* __restrict__ F, const float* __restrict__ Sl, const float* __restrict__ E,
    float* __restrict__ S_mid, float* __restrict__ S_last, int32_t n_mid, int32_t H) {
    constexpr size_t ST = 128 * 128;
    const int cb = blockIdx.x & 7;
    const int bh = blockIdx.x >> 3;
    const int b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x;
    const int j = tid & 15, rg = tid >> 4;   // column, row group (rows rg + 16 i)
    const int col = cb * MG_COLS + j;

    __shared__ __attribute__((aligned(16))) float sF[128 * MG_LDF];
    __shared__ float sS[128][MG_COLS];

    const size_t own = ((size_t)b * H + h) * ST;
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = E[own + (size_t)(rg + 16 * i) * 128 + col];

    for (int r = 0; r <= n_mid; ++r) {
        const size_t base = (((size_t)b * n_mid + r) * H + h) * ST;
        float* out = r < n_mid ? S_mid + base : S_last + own;
#pragma unroll
        for (int i = 0; i < 8; ++i) out[(size_t)(rg + 16 * i) * 128 + col] = s[i];
        if (r == n_mid) break;
        const float4* Fg = reinterpret_cast<const float4*>(F + base);
        for (int e = tid; e < 128 * 32; e += MG_THREADS)
            *reinterpret_cast<float4*>(&sF[(e >> 5) * MG_LDF + 4 * (e & 31)]) = Fg[e];
#pragma unroll
        for (int i = 0; i < 8; ++i) sS[rg + 16 * i][j] = s[i];
        __syncthreads();
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = Sl[base + (size_t)(rg + 16 * i) * 128 + col];
        for (int m = 0; m < 128; m += 4) {
            const float x0 = sS[m][j], x1 = sS[m + 1][j], x2 = sS[m + 2][j], x3 = sS[m + 3][j];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float4 f = *reinterpret_cast<const float4*>(&sF[(rg + 16 * i) * MG_LDF + m]);
                acc[i] = fmaf(f.x, x0, acc[i]);
                acc[i] = fmaf(f.y, x1, acc[i]);
                acc[i] = fmaf(f.z, x2, acc[i]);
                acc[i] = fmaf(f.w, x3, acc[i]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = acc[i];
    }
}

hipError_t launch_segment_merge(const float* F, const float* Sl, const float* E, float* S_mid,
                                float* S_last, int32_t B, int32_t n_mid, int32_t H,
                                hipStream_t stream) {
    dim3 grid((unsigned)((int64_t)B * H * 8)), block(MG_THREADS);
    hipLaunchKernelGGL(segment_merge_kernel, grid, block, 0, stream, F, Sl, E, S_mid, S_last, n_mid,
                       H);
    return hipGetLastError();
}

}  // namespace kda
