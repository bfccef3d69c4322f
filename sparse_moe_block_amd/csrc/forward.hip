// Forward, stages 0 and 3: the per-call schedule / activation staging, and the
// deterministic per-token weighted combine.
#include "common.h"

namespace fw {
namespace {

constexpr int kPrepThreads = 256;

// Block 0 turns expert_offsets into the list of active experts
// (expert, first row, rows) and the row-tile list -- each active expert's rows
// cut into tiles of at most tile_rows (the grouped GEMM's 128-row tiles, or the
// GEMV's token chunks) -- clamping anything out of range
// (FW_STATUS_BAD_OFFSETS).  The other blocks stage the token rows in fp16
// (bf16 values are exact in fp16), one 32-element block per thread over the
// T * H / 32 blocks of x, in the pair order both kernel families consume (see
// decode_pairs).
__global__ __launch_bounds__(kPrepThreads) void prepare_kernel(
    const int32_t *__restrict__ offsets, int E, int P, const void *__restrict__ x, int act_bf16,
    int H, int T, int tile_rows, int max_tiles, int4 *__restrict__ active, int4 *__restrict__ tiles,
    _Float16 *__restrict__ x16, float *__restrict__ xsum, int *__restrict__ split_cnt,
    WsHeader *__restrict__ hdr) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    if (blockIdx.x == 0) {
        // the GEMV's split-K arrival counters start every call at zero
        for (int i = tid; i < kSplitTiles; i += kPrepThreads) split_cnt[i] = 0;
        __shared__ int wsum_a[kPrepThreads / kWave], wsum_t[kPrepThreads / kWave];
        // each thread owns experts 2*tid and 2*tid+1
        int beg[2], cnt[2], na = 0, nt = 0;
        bool bad = false;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = 2 * tid + i;
            beg[i] = cnt[i] = 0;
            if (e < E) {
                int b = offsets[e], n = offsets[e + 1];
                if (e == 0 && b != 0) bad = true;
                if (b < 0 || b > P || n < b || n > P) bad = true;
                b = min(max(b, 0), P);
                n = min(max(n, b), P);
                beg[i] = b;
                cnt[i] = n - b;
                na += cnt[i] > 0;
                nt += (cnt[i] + tile_rows - 1) / tile_rows;
            }
        }
        if (bad) atomicOr(&hdr->status, FW_STATUS_BAD_OFFSETS);
        int ia = na, it = nt;   // inclusive scans
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int oa = __shfl_up(ia, off), ot = __shfl_up(it, off);
            if (lane >= off) {
                ia += oa;
                it += ot;
            }
        }
        if (lane == kWave - 1) {
            wsum_a[wave] = ia;
            wsum_t[wave] = it;
        }
        __syncthreads();
        int ba = 0, bt = 0;
        for (int w = 0; w < wave; ++w) {
            ba += wsum_a[w];
            bt += wsum_t[w];
        }
        int pa = ba + ia - na, pt = bt + it - nt;   // exclusive positions
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (cnt[i] > 0) {
                active[pa++] = int4{2 * tid + i, beg[i], cnt[i], 0};
                // bounded: overlapping (invalid) offsets can claim more
                for (int m = 0; m < cnt[i] && pt < max_tiles; m += tile_rows)
                    tiles[pt++] = int4{2 * tid + i, beg[i] + m, min(tile_rows, cnt[i] - m), 0};
            }
        }
        if (tid == kPrepThreads - 1) {
            hdr->n_active = ba + ia;
            hdr->n_tiles = min(bt + it, max_tiles);
        }
        return;
    }
    const long long idx = (long long)(blockIdx.x - 1) * kPrepThreads + tid;
    if (idx >= (long long)T * (H / 32)) return;
    const int t = (int)(idx / (H / 32)), b = (int)(idx % (H / 32));
    {
        float v[32];
        if (act_bf16) {
            const uint4 *src = (const uint4 *)((const uint16_t *)x + (size_t)t * H + 32 * b);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 raw = src[q];
                const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[8 * q + 2 * i] = __uint_as_float(wd[i] << 16);
                    v[8 * q + 2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
                }
            }
        } else {
            const float4 *src = (const float4 *)((const float *)x + (size_t)t * H + 32 * b);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 f = src[q];
                v[4 * q] = f.x;
                v[4 * q + 1] = f.y;
                v[4 * q + 2] = f.z;
                v[4 * q + 3] = f.w;
            }
        }
        uint32_t o[16];
#pragma unroll
        for (int pi = 0; pi < 16; ++pi) {
            const int m = pi >> 2, j = pi & 3;
            const int e0 = (j & 1 ? 16 : 0) + 4 * m + (j >> 1);
            const float sc = (j & 1) ? 0.0625f : 1.0f;
            o[pi] = __builtin_bit_cast(uint32_t, h2{(_Float16)(v[e0] * sc), (_Float16)(v[e0 + 2] * sc)});
        }
        uint4 *dst = (uint4 *)(x16 + (size_t)t * H + 32 * b);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = uint4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
        if (xsum) {
            // the block's sum of the staged fp16 values (unscaled), in pair
            // order: the min term of a Q4_K GEMV
            float sum = 0.f;
#pragma unroll
            for (int pi = 0; pi < 16; ++pi) {
                const h2 v = as_h2(o[pi]);
                const float sc = (pi & 1) ? 16.0f : 1.0f;
                sum += sc * (float)v[0];
                sum += sc * (float)v[1];
            }
            xsum[(size_t)t * (H / 32) + b] = sum;
        }
    }
}

// out[t][o] = sum_{j<k} w[t][j] * y[inv[t*k+j]][o]  (slot order)  + y_shared[t][o]
__global__ __launch_bounds__(256) void combine_kernel(
    const float *__restrict__ y, const float *__restrict__ ysh, const float *__restrict__ w,
    const int32_t *__restrict__ inv, float *__restrict__ out, int H, int k, int P,
    WsHeader *__restrict__ hdr) {
    const int t = blockIdx.y;
    const int o = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (o >= H) return;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    bool bad = false;
    for (int j = 0; j < k; ++j) {
        const int p = inv[(size_t)t * k + j];
        const float wj = w[(size_t)t * k + j];
        if ((unsigned)p >= (unsigned)P) {
            bad = true;
            continue;
        }
        const float4 v = *(const float4 *)(y + (size_t)p * H + o);
        acc.x = fmaf(wj, v.x, acc.x);
        acc.y = fmaf(wj, v.y, acc.y);
        acc.z = fmaf(wj, v.z, acc.z);
        acc.w = fmaf(wj, v.w, acc.w);
    }
    if (ysh) {
        const float4 v = *(const float4 *)(ysh + (size_t)t * H + o);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    *(float4 *)(out + (size_t)t * H + o) = acc;
    if (bad) atomicOr(&hdr->status, FW_STATUS_BAD_PAIR);
}

}  // namespace

hipError_t launch_prepare(const FwdArgs &a, hipStream_t s) {
    const int tile_rows = a.path == FW_PATH_GEMM ? (kUseGemm2 ? kGemm2BM : kGemmBM) : kGemvTokens;
    // the Q4_K GEMV needs the activation rows' block sums
    const bool sums = a.path == FW_PATH_GEMV &&
                      (a.d.expert_q == FW_Q4_K || (a.d.shared_ffn > 0 && a.d.shared_q == FW_Q4_K));
    const long long xblocks = (long long)a.T * (a.d.hidden / 32);
    prepare_kernel<<<1 + (int)((xblocks + kPrepThreads - 1) / kPrepThreads), kPrepThreads, 0, s>>>(
        a.offsets, a.d.n_experts, a.P, a.x, a.d.act_dtype == FW_BF16, a.d.hidden, a.T, tile_rows,
        a.L.max_tiles, (int4 *)(a.ws + a.L.active), (int4 *)(a.ws + a.L.tiles),
        (_Float16 *)(a.ws + a.L.x16), sums ? (float *)(a.ws + a.L.xsum) : nullptr,
        (int *)(a.ws + a.L.split_cnt), (WsHeader *)a.ws);
    return hipGetLastError();
}

hipError_t launch_combine(const FwdArgs &a, hipStream_t s) {
    const int H = a.d.hidden;
    const float *y = (const float *)(a.ws + a.L.y);
    const float *ysh = a.d.shared_ffn ? y + (size_t)a.P * H : nullptr;
    dim3 grid((H / 4 + 255) / 256, a.T);
    combine_kernel<<<grid, 256, 0, s>>>(y, ysh, a.topk_w, a.inv, a.out, H, a.d.top_k, a.P,
                                        (WsHeader *)a.ws);
    return hipGetLastError();
}

}  // namespace fw
