// Router: logits (x . W_r^T + b) and the per-token score / top-k / renormalise
// step.  (Flyweight 0.2.0 served-families table -- DeepSeek-shaped MoE; vOOM
// notes -- top-k as a per-request tunable; the plainest reading of both is the
// softmax- or sigmoid-scored top-k with renormalised weights.)
#include <math.h>

#include "common.h"

namespace fw {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 logits on MFMA.  A workgroup owns 16 tokens x (16*NE) experts; its four
// waves split the reduction dimension H into interleaved 32-wide steps and
// their partial tiles are summed in wave order through LDS.  bf16 x bf16
// products are exact in fp32 and accumulate in fp32.
//
// v_mfma_f32_16x16x32_bf16: lane l supplies A[m = l%16][k = 8*(l/16) .. +7] and
// B[k = 8*(l/16) .. +7][n = l%16]; it receives D[m = 4*(l/16) + i][n = l%16],
// i = 0..3.  A = x rows (tokens), B = W_r rows (experts), both read as 16
// contiguous bytes per lane.
template <int NE>
__global__ __launch_bounds__(256) void logits_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, float *__restrict__ logits, int T, int H, int E) {
    __shared__ f32x4 red[3][NE][kWave];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16 * NE;
    const int r = lane % 16, kq = (lane / 16) * 8;
    const int t = t0 + r;
    const bool tv = t < T;
    const uint16_t *xp = x + (size_t)(tv ? t : 0) * H + kq;
    const uint16_t *wp[NE];
    bool ev[NE];
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        const int e = e0 + 16 * n + r;
        ev[n] = e < E;
        wp[n] = wr + (size_t)(ev[n] ? e : 0) * H + kq;
    }
    f32x4 acc[NE];
#pragma unroll
    for (int n = 0; n < NE; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 zero = {};
    for (int k = wave * 32; k < H; k += 4 * 32) {
        bf16x8 a = tv ? *(const bf16x8 *)(xp + k) : zero;
#pragma unroll
        for (int n = 0; n < NE; ++n) {
            bf16x8 b = ev[n] ? *(const bf16x8 *)(wp[n] + k) : zero;
            acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[n], 0, 0, 0);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int n = 0; n < NE; ++n) red[wave - 1][n][lane] = acc[n];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        f32x4 v = acc[n];
#pragma unroll
        for (int w = 0; w < 3; ++w) v += red[w][n][lane];
        const int e = e0 + 16 * n + r;
        if (e >= E) continue;
        const float b = bias ? bias[e] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tt = t0 + 4 * (lane / 16) + i;
            if (tt < T) logits[(size_t)tt * E + e] = v[i] + b;
        }
    }
}

// fp32 logits (small layers): one thread per (token, expert), sequential sum.
__global__ __launch_bounds__(256) void logits_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    float *__restrict__ logits, int T, int H, int E) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * E) return;
    const int t = i / E, e = i % E;
    const float *xp = x + (size_t)t * H, *wp = wr + (size_t)e * H;
    float acc = 0.f;
    for (int h = 0; h < H; h += 4) {
        float4 a = *(const float4 *)(xp + h), b = *(const float4 *)(wp + h);
        acc = fmaf(a.x, b.x, acc);
        acc = fmaf(a.y, b.y, acc);
        acc = fmaf(a.z, b.z, acc);
        acc = fmaf(a.w, b.w, acc);
    }
    logits[i] = acc + (bias ? bias[e] : 0.f);
}

// One wavefront per token.  Lane l holds the logits of experts l, l+64, ...;
// k rounds of a wave-wide (value, index) arg-max with ties to the lower index
// pick the experts in descending order; lane j keeps slot j.  Renormalised
// weights: softmax -> exp(l_j - l_0) / sum over the slots (l_0 is the maximum);
// sigmoid -> s_j / sum s.
template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k, int score, int32_t *__restrict__ ids,
                                                   float *__restrict__ w) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    float v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        float l = e < E ? logits[(size_t)t * E + e] : -INFINITY;
        v[i] = (l == l) ? l : -INFINITY;   // NaN never outranks a number
    }
    uint32_t taken = 0;
    int my_e = 0;
    float my_l = 0.f;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + kWave * i;
            if (e < E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oe = __shfl_xor(be, off);
            if (ov > bv || (ov == bv && oe < be)) {
                bv = ov;
                be = oe;
            }
        }
        if ((be % kWave) == lane) taken |= 1u << (be / kWave);
        if (lane == j) {
            my_e = be;
            my_l = bv;
        }
    }
    const float l0 = __shfl(my_l, 0);
    float s = 0.f;
    if (lane < k) s = score == FW_SOFTMAX_RENORM ? expf(my_l - l0) : 1.0f / (1.0f + expf(-my_l));
    float sum = s;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        w[(size_t)t * k + lane] = s / sum;
    }
}

}  // namespace

hipError_t launch_logits(const fw_moe_desc &d, int T, const void *x, const void *wr,
                         const float *bias, float *logits, hipStream_t s) {
    const int H = d.hidden, E = d.n_experts;
    if (d.act_dtype == FW_F32) {
        const int n = T * E;
        logits_f32_kernel<<<(n + 255) / 256, 256, 0, s>>>((const float *)x, (const float *)wr,
                                                          bias, logits, T, H, E);
    } else if (E >= 64) {
        dim3 grid((T + 15) / 16, (E + 63) / 64);
        logits_bf16_kernel<4><<<grid, 256, 0, s>>>((const uint16_t *)x, (const uint16_t *)wr,
                                                   bias, logits, T, H, E);
    } else {
        dim3 grid((T + 15) / 16, (E + 15) / 16);
        logits_bf16_kernel<1><<<grid, 256, 0, s>>>((const uint16_t *)x, (const uint16_t *)wr,
                                                   bias, logits, T, H, E);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const fw_moe_desc &d, int T, const float *logits, int32_t *ids, float *w,
                       hipStream_t s) {
    const int E = d.n_experts, grid = (T + 3) / 4;
    const int epl = (E + kWave - 1) / kWave;
#define FW_TOPK(N)                                                                      \
    case N:                                                                             \
        topk_kernel<N><<<grid, 256, 0, s>>>(logits, T, E, d.top_k, d.score, ids, w); \
        break;
    switch (epl) {
        FW_TOPK(1)
        FW_TOPK(2)
        FW_TOPK(3)
        FW_TOPK(4)
        FW_TOPK(5)
        FW_TOPK(6)
        FW_TOPK(7)
        FW_TOPK(8)
        default:
            return hipErrorInvalidValue;
    }
#undef FW_TOPK
    return hipGetLastError();
}

}  // namespace fw
