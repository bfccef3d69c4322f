// Router: logits (x . W_r^T + b) and the per-token score / top-k / renormalise
// step.  (Flyweight 0.2.0 served-families table -- DeepSeek-shaped MoE; vOOM
// notes -- top-k as a per-request tunable; the plainest reading of both is the
// softmax- or sigmoid-scored top-k with renormalised weights.)
#include <math.h>

#include "common.h"
#include "stages.h"

namespace fw {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Up to this many tokens the bf16 logits run one wavefront per dot product.
constexpr int kLogitsDotMaxT = 16;

// bf16 logits on MFMA.  A workgroup owns 16*MT tokens x 16*NE experts; its NW
// waves split the reduction dimension H into interleaved 32-wide steps (wave
// w takes steps w, w + NW, ...), issue the loads of U steps before their
// MFMAs, and their partial tiles are summed in wave order through LDS.  bf16 x
// bf16 products are exact in fp32 and accumulate in fp32.
//
// Decode-sized batches use one 16 x 16 tile per workgroup and 16 waves, so the
// E x H router streams through E/16 workgroups with 16 loads in flight per
// wave; prefill-sized batches use 32 x 64 tiles and 4 waves, so each router
// row is re-read from L2 by fewer workgroups.
//
// v_mfma_f32_16x16x32_bf16: lane l supplies A[m = l%16][k = 8*(l/16) .. +7] and
// B[k = 8*(l/16) .. +7][n = l%16]; it receives D[m = 4*(l/16) + i][n = l%16],
// i = 0..3.  A = x rows (tokens), B = W_r rows (experts), both read as 16
// contiguous bytes per lane.
template <int MT, int NE, int NW, int U>
__global__ __launch_bounds__(NW *kWave) void logits_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, float *__restrict__ logits, int T, int H, int E) {
    __shared__ f32x4 red[NW - 1][MT * NE][kWave];
    const int wave = wave_id(), lane = threadIdx.x % kWave;
    const int t0 = blockIdx.x * 16 * MT, e0 = blockIdx.y * 16 * NE;
    const int r = lane % 16, kq = (lane / 16) * 8;
    const uint16_t *xp[MT], *wp[NE];
    bool tv[MT], ev[NE];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int t = t0 + 16 * m + r;
        tv[m] = t < T;
        xp[m] = x + (size_t)(tv[m] ? t : 0) * H + kq;
    }
#pragma unroll
    for (int n = 0; n < NE; ++n) {
        const int e = e0 + 16 * n + r;
        ev[n] = e < E;
        wp[n] = wr + (size_t)(ev[n] ? e : 0) * H + kq;
    }
    f32x4 acc[MT][NE];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NE; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 zero = {};
    const int steps = H / 32;
    for (int s0 = wave; s0 < steps; s0 += NW * U) {
        bf16x8 a[U][MT], b[U][NE];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = s0 + u * NW;
            const bool in = s < steps;
#pragma unroll
            for (int m = 0; m < MT; ++m)
                a[u][m] = (in && tv[m]) ? *(const bf16x8 *)(xp[m] + 32 * s) : zero;
#pragma unroll
            for (int n = 0; n < NE; ++n)
                b[u][n] = (in && ev[n]) ? *(const bf16x8 *)(wp[n] + 32 * s) : zero;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int n = 0; n < NE; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][m], b[u][n],
                                                                        acc[m][n], 0, 0, 0);
    }
    if (wave > 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int n = 0; n < NE; ++n) red[wave - 1][m * NE + n][lane] = acc[m][n];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NE; ++n) {
            f32x4 v = acc[m][n];
            for (int w = 0; w < NW - 1; ++w) v += red[w][m * NE + n][lane];
            const int e = e0 + 16 * n + r;
            if (e >= E) continue;
            const float b = bias ? bias[e] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tt = t0 + 16 * m + 4 * (lane / 16) + i;
                if (tt < T) logits[(size_t)tt * E + e] = v[i] + b;
            }
        }
}

// bf16 logits for a few tokens: one wavefront per (token, expert) dot product,
// so the E x H router spreads over E * T wavefronts (a 16-token, 128-expert
// batch: 512 workgroups) instead of E / 16 workgroups.  Each lane loads NC
// 16-byte chunks of the router row and of the token row at once (all in
// flight together), sums their exact bf16 x bf16 products in fp32 in element
// order, and the wavefront's lanes are added in a fixed butterfly order.
template <int NC>
__global__ __launch_bounds__(256) void logits_dot_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, float *__restrict__ logits, int T, int H, int E) {
    const int lane = threadIdx.x % kWave;
    const int pair = blockIdx.x * 4 + wave_id();   // (token, expert)
    if (pair >= T * E) return;
    const int t = pair / E, e = pair % E;
    const uint4 *wp = (const uint4 *)(wr + (size_t)e * H) + lane;
    const uint4 *xp = (const uint4 *)(x + (size_t)t * H) + lane;
    uint4 wv[NC], xv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        wv[c] = wp[c * kWave];
        xv[c] = xp[c * kWave];
    }
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const uint32_t a[4] = {wv[c].x, wv[c].y, wv[c].z, wv[c].w};
        const uint32_t b[4] = {xv[c].x, xv[c].y, xv[c].z, xv[c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), acc);
            acc = fmaf(__uint_as_float(a[i] & 0xFFFF0000u), __uint_as_float(b[i] & 0xFFFF0000u),
                       acc);
        }
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) logits[(size_t)t * E + e] = acc + (bias ? bias[e] : 0.f);
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

template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k, int score, int32_t *__restrict__ ids,
                                                   float *__restrict__ w) {
    const int t = blockIdx.x * 4 + wave_id();
    if (t >= T) return;
    topk_token<EPL>(logits, t, E, k, score, ids, w, nullptr);
}

}  // namespace

hipError_t launch_logits(const fw_moe_desc &d, int T, const void *x, const void *wr,
                         const float *bias, float *logits, hipStream_t s) {
    const int H = d.hidden, E = d.n_experts;
    const uint16_t *xb = (const uint16_t *)x, *wb = (const uint16_t *)wr;
    if (d.act_dtype == FW_F32) {
        const int n = T * E;
        logits_f32_kernel<<<(n + 255) / 256, 256, 0, s>>>((const float *)x, (const float *)wr,
                                                          bias, logits, T, H, E);
    } else if (T <= kLogitsDotMaxT && H % 512 == 0 && H <= 512 * 16) {
        // 16-byte chunks per lane: H / 512
        const int blocks = (T * E + 3) / 4;
        switch (H / 512) {
#define FW_LD(NC)                                                                              \
    case NC:                                                                                   \
        logits_dot_kernel<NC><<<blocks, 256, 0, s>>>(xb, wb, bias, logits, T, H, E);           \
        break;
            FW_LD(1) FW_LD(2) FW_LD(3) FW_LD(4) FW_LD(5) FW_LD(6) FW_LD(7) FW_LD(8)
            FW_LD(9) FW_LD(10) FW_LD(11) FW_LD(12) FW_LD(13) FW_LD(14) FW_LD(15) FW_LD(16)
#undef FW_LD
            default:
                return hipErrorInvalidValue;
        }
    } else if (T <= kLogitsTileMaxT) {
        dim3 grid((T + 15) / 16, (E + 15) / 16);
        logits_bf16_kernel<1, 1, 16, 4><<<grid, 16 * kWave, 0, s>>>(xb, wb, bias, logits, T, H, E);
    } else if (E >= 64 && (long long)((T + 63) / 64) * ((E + 63) / 64) >= 256) {
        // enough 64 x 64 tiles for every CU: each x row is read by E/64
        // workgroups and each router row by T/64 (32 x 64 tiles: twice as
        // many router reads and two rounds of workgroups)
        dim3 grid((T + 63) / 64, (E + 63) / 64);
        logits_bf16_kernel<4, 4, 4, 2><<<grid, 4 * kWave, 0, s>>>(xb, wb, bias, logits, T, H, E);
    } else if (E >= 64 && (long long)((T + 31) / 32) * ((E + 63) / 64) >= 512) {
        dim3 grid((T + 31) / 32, (E + 63) / 64);
        logits_bf16_kernel<2, 4, 4, 2><<<grid, 4 * kWave, 0, s>>>(xb, wb, bias, logits, T, H, E);
    } else if (E >= 32) {
        // fewer than 512 of the 32 x 64 tiles: 32 x 32 tiles over 8 wavefronts
        // keep more of the CUs busy (T = 2048, E = 128: 20 -> 13 us)
        dim3 grid((T + 31) / 32, (E + 31) / 32);
        logits_bf16_kernel<2, 2, 8, 2><<<grid, 8 * kWave, 0, s>>>(xb, wb, bias, logits, T, H, E);
    } else {
        dim3 grid((T + 31) / 32, (E + 15) / 16);
        logits_bf16_kernel<2, 1, 4, 4><<<grid, 4 * kWave, 0, s>>>(xb, wb, bias, logits, T, H, E);
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
