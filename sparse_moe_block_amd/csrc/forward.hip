// Forward, stages 0 and 3: the per-call schedule / activation staging, and the
// deterministic per-token weighted combine.
#include "common.h"
#include "stages.h"

namespace fw {
namespace {

// Block 0 turns expert_offsets into the list of active experts
// (expert, first row, rows) and the row-tile list -- each active expert's rows
// cut into tiles of at most tile_rows (the grouped GEMM's 128-row tiles, or the
// GEMV's token chunks) -- clamping anything out of range
// (FW_STATUS_BAD_OFFSETS).  In the other blocks each wavefront stages one
// token row in fp16, scaled by its power-of-two exponent (stage_x_row), in
// the pair order both kernel families consume (see decode_pairs).
__global__ __launch_bounds__(kPrepThreads) void prepare_kernel(
    const int32_t *__restrict__ offsets, int E, int P, const void *__restrict__ x, int act_bf16,
    int H, int T, int tile_rows, int max_tiles, int4 *__restrict__ active, int4 *__restrict__ tiles,
    _Float16 *__restrict__ x16, float *__restrict__ xsum, int32_t *__restrict__ xe,
    int *__restrict__ split_cnt, WsHeader *__restrict__ hdr, TileCost cost) {
    if (blockIdx.x == 0) {
        build_schedule(offsets, E, P, tile_rows, max_tiles, active, tiles, split_cnt, hdr,
                       cost);
        return;
    }
    const int t = (blockIdx.x - 1) * (kPrepThreads / kWave) + wave_id();
    if (t >= T) return;
    stage_x_row(x, act_bf16, H, t, x16, xsum, xe, hdr);
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
    if (a.d.act_quant == FW_ACT_MXFP8) return launch_prepare_mx8(a, s);
    if (a.d.act_quant == FW_ACT_INT8) return launch_prepare_i8(a, s);
    const int tile_rows = a.path == FW_PATH_GEMM ? gemm_tile_rows(a.d.expert_q) : kGemvTokens;
    // the Q4_K GEMV needs the activation rows' block sums
    const bool sums = a.path == FW_PATH_GEMV &&
                      (a.d.expert_q == FW_Q4_K || (a.d.shared_ffn > 0 && a.d.shared_q == FW_Q4_K));
    constexpr int rows_per_block = kPrepThreads / kWave;   // one wavefront per token row
    prepare_kernel<<<1 + (a.T + rows_per_block - 1) / rows_per_block, kPrepThreads, 0, s>>>(
        a.offsets, a.d.n_experts, a.P, a.x, a.d.act_dtype == FW_BF16, a.d.hidden, a.T, tile_rows,
        a.L.max_tiles, (int4 *)(a.ws + a.L.active), (int4 *)(a.ws + a.L.tiles),
        (_Float16 *)(a.ws + a.L.x16), sums ? (float *)(a.ws + a.L.xsum) : nullptr,
        (int32_t *)(a.ws + a.L.xe), (int *)(a.ws + a.L.split_cnt), (WsHeader *)a.ws,
        gemm_tile_cost(a.d.expert_q));
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
