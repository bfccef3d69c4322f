// Forward, GEMV family (decode-sized batches): dequant-fused expert projections
// that read each active expert's blocks once.  Decode is bandwidth-bound (the
// pages' runtime measures it in spilled bytes per token -- Flyweight 0.2.0
// "Quantization"), so these kernels are built around HBM streaming:
//
//  - one lane per weight row: a wavefront owns 64 consecutive rows of one
//    expert and walks them along the reduction dimension in 256-element units
//    (8 GGUF blocks, 16-byte aligned), loaded as dwordx4s and decoded in
//    registers; the next unit is in flight while the current one is consumed;
//  - the activations of the expert's tokens are the same for every lane, so
//    they are read with scalar loads and enter each FMA as a scalar operand;
//  - codes are turned into floats without their offset (Q4_0: q, Q8_0: q+128)
//    and the offset is removed once per block with the activation block sum;
//    the fp16 block scale is applied once per block;
//  - the reduction dimension is split over S wavefronts of a workgroup (more
//    loads in flight for small batches); the partial sums meet in LDS and are
//    added in wavefront order, so results are deterministic.
// Gate and up rows of the same feature share the lane, so SiLU(g)*u is formed
// in registers (the fused gate/up pass that shares each activation load:
// Flyweight 0.2.0 "Current limitations").
#include <math.h>

#include "common.h"

namespace fw {
namespace {

constexpr int NT = kGemvTokens;

// Activations are read through the constant address space: they are not
// written while a GEMV kernel runs, and uniform loads from it become scalar
// loads (s_load), so every lane's FMA takes them as a scalar operand.
typedef __attribute__((address_space(4))) const float cfloat;

template <int Q> struct Unit {
    uint4 v[QT<Q>::kUnitX4];
};

template <int Q>
__device__ __forceinline__ void load_unit(Unit<Q> &b, const uint8_t *row, int u) {
    const uint4 *p = (const uint4 *)(row + (size_t)u * QT<Q>::kUnitBytes);
#pragma unroll
    for (int i = 0; i < QT<Q>::kUnitX4; ++i) b.v[i] = p[i];
}

// acc[n] += sum over unit u of row . in_n, for the nt (uniform) token rows
// whose activation rows start at in[n] (fp32) and block sums at ins[n].
template <int Q, int B>
__device__ __forceinline__ void consume_block(const uint32_t *w, int u, cfloat *const *in,
                                              cfloat *const *ins, int nt, float *acc) {
    float d, c[32];
    decode_block<Q, B>(w, d, c);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        if (n < nt) {
            cfloat *xp = in[n] + u * kUnit + 32 * B;
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) p = fmaf(c[i], xp[i], p);
            acc[n] = fmaf(d, p - QT<Q>::kOffset * ins[n][u * 8 + B], acc[n]);
        }
    }
}

template <int Q>
__device__ __forceinline__ void consume_unit(const Unit<Q> &b, int u, cfloat *const *in,
                                             cfloat *const *ins, int nt, float *acc) {
    uint32_t w[4 * QT<Q>::kUnitX4];
#pragma unroll
    for (int i = 0; i < QT<Q>::kUnitX4; ++i) {
        w[4 * i] = b.v[i].x;
        w[4 * i + 1] = b.v[i].y;
        w[4 * i + 2] = b.v[i].z;
        w[4 * i + 3] = b.v[i].w;
    }
    consume_block<Q, 0>(w, u, in, ins, nt, acc);
    consume_block<Q, 1>(w, u, in, ins, nt, acc);
    consume_block<Q, 2>(w, u, in, ins, nt, acc);
    consume_block<Q, 3>(w, u, in, ins, nt, acc);
    consume_block<Q, 4>(w, u, in, ins, nt, acc);
    consume_block<Q, 5>(w, u, in, ins, nt, acc);
    consume_block<Q, 6>(w, u, in, ins, nt, acc);
    consume_block<Q, 7>(w, u, in, ins, nt, acc);
}

// Partial sums of waves 1..S-1 meet wave 0's in LDS, added in wave order.
// Returns true in the wave that holds the total.
template <int NV>
__device__ __forceinline__ bool reduce_waves(float (*acc)[NT], float (*red)[NV][NT][kWave],
                                             int S, int wave, int lane) {
    if (S == 1) return true;
    if (wave > 0) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int n = 0; n < NT; ++n) red[wave - 1][v][n][lane] = acc[v][n];
    }
    __syncthreads();
    if (wave == 0) {
        for (int w = 0; w < S - 1; ++w)
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[v][n] += red[w][v][n][lane];
    }
    return wave == 0;
}

constexpr int kMaxSplit = 4;

// Gate and up projections of one 64-row tile of one expert (or of the shared
// expert) for the expert's rows [rb, rb + rc) of the sorted pair list; writes
// a = SiLU(g) * u and its 32-element block sums.
template <int Q>
__global__ __launch_bounds__(kWave *kMaxSplit) void gemv_gate_up_kernel(
    const uint8_t *__restrict__ wg, const uint8_t *__restrict__ wu,
    const int4 *__restrict__ active, WsHeader *__restrict__ hdr,
    const int32_t *__restrict__ sorted, const float *__restrict__ x32,
    const float *__restrict__ xs, float *__restrict__ h, float *__restrict__ hs, int H, int F,
    int k, int P, int tiles_per_group, int shared, int S) {
    __shared__ float red[kMaxSplit - 1][2][NT][kWave];
    const int g = blockIdx.x / tiles_per_group, tile = blockIdx.x % tiles_per_group;
    int rb = 0, rc = P / k;
    const uint8_t *rg = wg, *ru = wu;
    if (!shared) {
        if (g >= ld_const(&hdr->n_active)) return;
        const int4 ex = ld_const(active + g);   // (expert, first row, rows)
        const size_t esz = (size_t)F * (H / 32) * QT<Q>::kBlockBytes;
        rg += ex.x * esz;
        ru += ex.x * esz;
        rb = ex.y;
        rc = ex.z;
    }
    const int wave = wave_id(), lane = threadIdx.x % kWave;
    const int f = tile * kWave + lane;
    const size_t rowbytes = (size_t)(H / 32) * QT<Q>::kBlockBytes;
    rg += (size_t)f * rowbytes;
    ru += (size_t)f * rowbytes;
    const int U = H / kUnit, u0 = wave * U / S, u1 = (wave + 1) * U / S;
    for (int c0 = 0; c0 < rc; c0 += NT) {
        const int nt = min(NT, rc - c0);
        cfloat *in[NT], *ins[NT];
        bool bad = false;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int r = rb + c0 + min(n, nt - 1);
            int t = r;
            if (!shared) {
                const int q = ld_const(sorted + r);
                if ((unsigned)q >= (unsigned)P) {
                    bad = true;
                    t = 0;
                } else {
                    t = q / k;
                }
            }
            in[n] = (cfloat *)(x32 + (size_t)t * H);
            ins[n] = (cfloat *)(xs + (size_t)t * (H / 32));
        }
        if (bad && threadIdx.x == 0) atomicOr(&hdr->status, FW_STATUS_BAD_PAIR);
        float acc[2][NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[0][n] = acc[1][n] = 0.f;
        Unit<Q> A, B;
        load_unit<Q>(A, rg, u0);
        load_unit<Q>(B, ru, u0);
        for (int u = u0; u < u1; ++u) {
            consume_unit<Q>(A, u, in, ins, nt, acc[0]);
            if (u + 1 < u1) load_unit<Q>(A, rg, u + 1);
            consume_unit<Q>(B, u, in, ins, nt, acc[1]);
            if (u + 1 < u1) load_unit<Q>(B, ru, u + 1);
        }
        if (reduce_waves<2>(acc, red, S, wave, lane)) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if (n < nt) {
                    const float gv = acc[0][n], up = acc[1][n];
                    const float a = gv / (1.0f + expf(-gv)) * up;
                    const int r = rb + c0 + n;
                    h[(size_t)r * F + f] = a;
                    float sum = a;
#pragma unroll
                    for (int off = 16; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
                    if ((lane & 31) == 0) hs[(size_t)r * (F / 32) + f / 32] = sum;
                }
            }
        }
        if (S > 1) __syncthreads();   // red[] is reused by the next chunk
    }
}

// Down projection of one 64-row tile (outputs o) of one expert (or of the
// shared expert) for rows [rb, rb + rc): y[r][o] = W_down[o] . a[r].
template <int Q>
__global__ __launch_bounds__(kWave *kMaxSplit) void gemv_down_kernel(
    const uint8_t *__restrict__ wd, const int4 *__restrict__ active,
    const WsHeader *__restrict__ hdr, const float *__restrict__ h,
    const float *__restrict__ hs, float *__restrict__ y, int H, int F, int P_rows,
    int tiles_per_group, int shared, int S) {
    __shared__ float red[kMaxSplit - 1][1][NT][kWave];
    const int g = blockIdx.x / tiles_per_group, tile = blockIdx.x % tiles_per_group;
    int rb = 0, rc = P_rows;
    const uint8_t *row = wd;
    if (!shared) {
        if (g >= ld_const(&hdr->n_active)) return;
        const int4 ex = ld_const(active + g);
        row += ex.x * ((size_t)H * (F / 32) * QT<Q>::kBlockBytes);
        rb = ex.y;
        rc = ex.z;
    }
    const int wave = wave_id(), lane = threadIdx.x % kWave;
    const int o = tile * kWave + lane;
    row += (size_t)o * ((size_t)(F / 32) * QT<Q>::kBlockBytes);
    const int U = F / kUnit, u0 = wave * U / S, u1 = (wave + 1) * U / S;
    for (int c0 = 0; c0 < rc; c0 += NT) {
        const int nt = min(NT, rc - c0);
        cfloat *in[NT], *ins[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int r = rb + c0 + min(n, nt - 1);
            in[n] = (cfloat *)(h + (size_t)r * F);
            ins[n] = (cfloat *)(hs + (size_t)r * (F / 32));
        }
        float acc[1][NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[0][n] = 0.f;
        Unit<Q> A, B;
        load_unit<Q>(A, row, u0);
        if (u0 + 1 < u1) load_unit<Q>(B, row, u0 + 1);
        for (int u = u0; u < u1; u += 2) {
            consume_unit<Q>(A, u, in, ins, nt, acc[0]);
            if (u + 2 < u1) load_unit<Q>(A, row, u + 2);
            if (u + 1 < u1) {
                consume_unit<Q>(B, u + 1, in, ins, nt, acc[0]);
                if (u + 3 < u1) load_unit<Q>(B, row, u + 3);
            }
        }
        if (reduce_waves<1>(acc, red, S, wave, lane)) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
                if (n < nt) y[(size_t)(rb + c0 + n) * H + o] = acc[0][n];
        }
        if (S > 1) __syncthreads();
    }
}

// Wavefronts per workgroup: the reduction dimension is split in S contiguous
// ranges of whole 256-element units.
int pick_split(int units) {
    for (int s : {4, 3, 2})
        if (units % s == 0) return s;
    return 1;
}

template <int Q>
void gate_up_launch(const FwdArgs &a, const uint8_t *wg, const uint8_t *wu, int F, int groups,
                    int shared, float *h, float *hs, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const int S = pick_split(d.hidden / kUnit), tpg = F / kWave;
    gemv_gate_up_kernel<Q><<<groups * tpg, kWave * S, 0, s>>>(
        wg, wu, (const int4 *)(a.ws + a.L.active), (WsHeader *)a.ws, a.sorted,
        (const float *)(a.ws + a.L.x32), (const float *)(a.ws + a.L.xs), h, hs, d.hidden, F,
        d.top_k, a.P, tpg, shared, S);
}

template <int Q>
void down_launch(const FwdArgs &a, const uint8_t *wd, int F, int groups, int shared,
                 const float *h, const float *hs, float *y, int rows, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const int S = pick_split(F / kUnit), tpg = d.hidden / kWave;
    gemv_down_kernel<Q><<<groups * tpg, kWave * S, 0, s>>>(
        wd, (const int4 *)(a.ws + a.L.active), (const WsHeader *)a.ws, h, hs, y, d.hidden, F,
        rows, tpg, shared, S);
}

}  // namespace

hipError_t launch_gemv_gate_up(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    float *h = (float *)(a.ws + a.L.h), *hs = (float *)(a.ws + a.L.hs);
    const int groups = std::min(d.n_experts, a.P);
    if (d.expert_q == FW_Q4_0)
        gate_up_launch<FW_Q4_0>(a, a.wg, a.wu, d.ffn, groups, 0, h, hs, s);
    else
        gate_up_launch<FW_Q8_0>(a, a.wg, a.wu, d.ffn, groups, 0, h, hs, s);
    if (d.shared_ffn > 0) {
        float *hsh = h + (size_t)a.P * d.ffn, *hssh = hs + (size_t)a.P * (d.ffn / 32);
        if (d.shared_q == FW_Q4_0)
            gate_up_launch<FW_Q4_0>(a, a.sg, a.su, d.shared_ffn, 1, 1, hsh, hssh, s);
        else
            gate_up_launch<FW_Q8_0>(a, a.sg, a.su, d.shared_ffn, 1, 1, hsh, hssh, s);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_down(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const float *h = (const float *)(a.ws + a.L.h), *hs = (const float *)(a.ws + a.L.hs);
    float *y = (float *)(a.ws + a.L.y);
    const int groups = std::min(d.n_experts, a.P);
    if (d.expert_q == FW_Q4_0)
        down_launch<FW_Q4_0>(a, a.wd, d.ffn, groups, 0, h, hs, y, a.P, s);
    else
        down_launch<FW_Q8_0>(a, a.wd, d.ffn, groups, 0, h, hs, y, a.P, s);
    if (d.shared_ffn > 0) {
        const float *hsh = h + (size_t)a.P * d.ffn, *hssh = hs + (size_t)a.P * (d.ffn / 32);
        float *ysh = y + (size_t)a.P * d.hidden;
        if (d.shared_q == FW_Q4_0)
            down_launch<FW_Q4_0>(a, a.sd, d.shared_ffn, 1, 1, hsh, hssh, ysh, a.T, s);
        else
            down_launch<FW_Q8_0>(a, a.sd, d.shared_ffn, 1, 1, hsh, hssh, ysh, a.T, s);
    }
    return hipGetLastError();
}

}  // namespace fw
