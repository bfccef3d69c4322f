// The fused decode front end of fw_moe_layer: top-k, permutation and the
// forward's staging in one launch, for batches the GEMV family serves.
//
// Separately these are three kernels (top-k, permute, prepare), each a few
// microseconds of mostly launch latency at decode sizes.  Here block 0 runs
// them back to back -- one wavefront per token for the top-k (ids also kept
// in LDS), the one-workgroup counting sort over those LDS ids, then the
// active-expert list and row tiles from the offsets it has just written --
// while the other blocks stage the token rows in fp16, which does not depend
// on the routing.  Every stage is the same device code as in the separate
// kernels, so the results are bit for bit the same.
#include "common.h"
#include "stages.h"

namespace fw {
namespace {

template <int EPL>
__global__ __launch_bounds__(kPermThreads) void decode_front_kernel(
    const float *__restrict__ logits, int T, int E, int k, int score, int32_t *__restrict__ ids,
    float *__restrict__ w, int32_t *__restrict__ offsets, int32_t *__restrict__ sorted,
    int32_t *__restrict__ inv, const void *__restrict__ x, int act_bf16, int H, int tile_rows,
    int max_tiles, int4 *__restrict__ active, int4 *__restrict__ tiles,
    _Float16 *__restrict__ x16, float *__restrict__ xsum, int *__restrict__ split_cnt,
    WsHeader *__restrict__ hdr) {
    if (blockIdx.x == 0) {
        __shared__ int32_t s_ids[kPermOneBlockMaxP];   // T * k <= kPermOneBlockMaxP
        for (int t = wave_id(); t < T; t += kPermWaves)
            topk_token<EPL>(logits, t, E, k, score, ids, w, s_ids);
        __syncthreads();
        permute_block(s_ids, T * k, E, offsets, sorted, inv, hdr);
        // the offsets written above are read back by this block only; the
        // barrier orders the global writes before those reads
        __syncthreads();
        build_schedule(offsets, E, T * k, tile_rows, max_tiles, active, tiles, split_cnt, hdr);
        return;
    }
    const long long idx = (long long)(blockIdx.x - 1) * kPermThreads + threadIdx.x;
    if (idx >= (long long)T * (H / 32)) return;
    stage_x_block(x, act_bf16, H, (int)(idx / (H / 32)), (int)(idx % (H / 32)), x16, xsum);
}

}  // namespace

bool decode_front_fits(const fw_moe_desc &d, int T, int path) {
    return path == FW_PATH_GEMV && T >= 1 && (long long)T * d.top_k <= kPermOneBlockMaxP;
}

hipError_t launch_decode_front(const FwdArgs &a, const float *logits, int32_t *ids, float *w,
                               int32_t *offsets, int32_t *sorted, int32_t *inv, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    if (!decode_front_fits(d, a.T, a.path)) return hipErrorInvalidValue;
    const bool sums = d.expert_q == FW_Q4_K || (d.shared_ffn > 0 && d.shared_q == FW_Q4_K);
    const long long xblocks = (long long)a.T * (d.hidden / 32);
    const int grid = 1 + (int)((xblocks + kPermThreads - 1) / kPermThreads);
    const int epl = (d.n_experts + kWave - 1) / kWave;
#define FW_FRONT(N)                                                                            \
    case N:                                                                                    \
        decode_front_kernel<N><<<grid, kPermThreads, 0, s>>>(                                  \
            logits, a.T, d.n_experts, d.top_k, d.score, ids, w, offsets, sorted, inv, a.x,     \
            d.act_dtype == FW_BF16, d.hidden, kGemvTokens, a.L.max_tiles,                      \
            (int4 *)(a.ws + a.L.active), (int4 *)(a.ws + a.L.tiles),                           \
            (_Float16 *)(a.ws + a.L.x16), sums ? (float *)(a.ws + a.L.xsum) : nullptr,         \
            (int *)(a.ws + a.L.split_cnt), (WsHeader *)a.ws);                                  \
        break;
    switch (epl) {
        FW_FRONT(1)
        FW_FRONT(2)
        FW_FRONT(3)
        FW_FRONT(4)
        FW_FRONT(5)
        FW_FRONT(6)
        FW_FRONT(7)
        FW_FRONT(8)
        default:
            return hipErrorInvalidValue;
    }
#undef FW_FRONT
    return hipGetLastError();
}

}  // namespace fw
