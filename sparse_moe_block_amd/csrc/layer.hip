// The fused decode front end of fw_moe_layer: top-k, permutation and the
// forward's staging in one launch, for batches the GEMV family serves.
//
// Separately these are three kernels (top-k, permute, prepare), each a few
// microseconds of mostly launch latency at decode sizes.  Here block 0 runs
// them back to back -- one wavefront per token for the top-k (ids also kept
// in LDS), then the counting sort over those LDS ids and the active-expert
// list and row tiles -- while the other blocks stage the token rows in fp16
// (one wavefront per row), which does not depend on the routing.  Up to 64 pairs one wavefront sorts
// and schedules without workgroup barriers; above that the block runs the
// same workgroup sort and schedule as the separate kernels.  The sort is
// stable and the schedule is in expert order either way, so the results are
// bit for bit those of the three kernels.
#include "common.h"
#include "stages.h"

namespace fw {
namespace {

// Pairs up to which one wavefront sorts and schedules.  One 64-pair chunk:
// decode T = 1 and 4 (8 and 32 pairs) gain about 1 us over the workgroup
// sort; at 256 pairs (DeepSeek T = 32) the wavefront's four chunks in turn
// took 2 us longer than the workgroup sort.
constexpr int kSmallP = 64;

// The stable counting sort and the row-tile schedule of up to kSmallP pairs
// by one wavefront, with no workgroup barrier (written for any number of
// 64-pair chunks, used for one): the same offsets, sorted list,
// inverse, active-expert list and tiles as permute_block + build_schedule.
// s_cnt [kMaxExperts] LDS starts at zero.  Lanes holding the same expert in a
// 64-pair chunk find each other with ballots over the 9 id bits; the group's
// lowest lane updates that expert's LDS count (or cursor), so no two lanes
// write one address in an instruction, and the wavefront's LDS operations
// take effect in program order.  Lane l owns experts 8l .. 8l + 7 (E <= 512)
// for the scan and the schedule.
__device__ __forceinline__ void small_sort_schedule(
    const int32_t *s_ids, int P, int E, int tile_rows, int max_tiles, int *s_cnt,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted, int32_t *__restrict__ inv,
    int4 *__restrict__ active, int4 *__restrict__ tiles, WsHeader *__restrict__ hdr) {
    const int lane = threadIdx.x % kWave;
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    auto group = [&](int e, bool valid) {   // lanes of this chunk holding expert e
        unsigned long long peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 9; ++b) {
            const bool bit = valid && ((e >> b) & 1);
            const unsigned long long m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        return peers;
    };
    // 1. counts
    bool bad = false;
    for (int c = 0; c * kWave < P; ++c) {
        const int q = c * kWave + lane;
        const int e = q < P ? s_ids[q] : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        if (q < P && !valid) bad = true;
        const unsigned long long peers = group(e, valid);
        if (valid && (peers & lt_mask) == 0) s_cnt[e] += __popcll(peers);
    }
    if (bad) atomicOr(&hdr->status, FW_STATUS_BAD_EXPERT_ID);
    // 2. exclusive scan -> offsets; the counts become cursors
    int cnt8[8], loc = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = 8 * lane + i;
        cnt8[i] = e < E ? s_cnt[e] : 0;
        loc += cnt8[i];
    }
    int incl = loc;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    const int total = __shfl(incl, kWave - 1);
    int beg8[8], run = incl - loc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = 8 * lane + i;
        beg8[i] = run;
        if (e < E) {
            offsets[e] = run;
            s_cnt[e] = run;
        }
        run += cnt8[i];
    }
    if (lane == 0) offsets[E] = total;
    // 3. positions: cursor + rank among the chunk's lanes of the same expert
    for (int c = 0; c * kWave < P; ++c) {
        const int q = c * kWave + lane;
        const int e = q < P ? s_ids[q] : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        const unsigned long long peers = group(e, valid);
        const int rank = __popcll(peers & lt_mask);
        if (valid) {
            const int pos = s_cnt[e] + rank;   // < offsets[e + 1] <= P
            if ((unsigned)pos < (unsigned)P) {
                sorted[pos] = q;
                inv[q] = pos;
            }
        } else if (q < P) {
            inv[q] = -1;
        }
        if (valid && rank == 0) s_cnt[e] += __popcll(peers);
    }
    for (int p = total + lane; p < P; p += kWave) sorted[p] = -1;
    // 4. active experts and row tiles, in expert order
    int na = 0, nt = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        na += cnt8[i] > 0;
        nt += (cnt8[i] + tile_rows - 1) / tile_rows;
    }
    int ia = na, it = nt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int oa = __shfl_up(ia, off), ot = __shfl_up(it, off);
        if (lane >= off) {
            ia += oa;
            it += ot;
        }
    }
    int pa = ia - na, pt = it - nt;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (cnt8[i] > 0) {
            const int e = 8 * lane + i;
            active[pa++] = int4{e, beg8[i], cnt8[i], 0};
            for (int m = 0; m < cnt8[i] && pt < max_tiles; m += tile_rows)
                tiles[pt++] = int4{e, beg8[i] + m, min(tile_rows, cnt8[i] - m), 0};
        }
    }
    if (lane == kWave - 1) {
        hdr->n_active = ia;
        hdr->n_tiles = min(it, max_tiles);
    }
}

// SMALL (T * k <= kSmallP): block 0's wavefront 0 sorts and schedules alone
// after the top-k; otherwise the whole block runs the workgroup sort and
// schedule.
template <int EPL, bool SMALL>
__global__ __launch_bounds__(kPermThreads) void decode_front_kernel(
    const float *__restrict__ logits, int T, int E, int k, int score, int32_t *__restrict__ ids,
    float *__restrict__ w, int32_t *__restrict__ offsets, int32_t *__restrict__ sorted,
    int32_t *__restrict__ inv, const void *__restrict__ x, int act_bf16, int H, int tile_rows,
    int max_tiles, int4 *__restrict__ active, int4 *__restrict__ tiles,
    _Float16 *__restrict__ x16, float *__restrict__ xsum, int32_t *__restrict__ xe,
    int *__restrict__ split_cnt, WsHeader *__restrict__ hdr) {
    if (blockIdx.x == 0) {
        __shared__ int32_t s_ids[SMALL ? kSmallP : kPermOneBlockMaxP];   // T * k fits
        if constexpr (SMALL) {
            __shared__ int s_cnt[kMaxExperts];
            for (int i = threadIdx.x; i < kMaxExperts; i += kPermThreads) s_cnt[i] = 0;
            // the GEMV's split-K arrival counters start every call at zero
            for (int i = threadIdx.x; i < kSplitTiles; i += kPermThreads) split_cnt[i] = 0;
            for (int t = wave_id(); t < T; t += kPermWaves)
                topk_token<EPL>(logits, t, E, k, score, ids, w, s_ids);
            __syncthreads();
            if (wave_id() == 0)
                small_sort_schedule(s_ids, T * k, E, tile_rows, max_tiles, s_cnt, offsets,
                                    sorted, inv, active, tiles, hdr);
        } else {
            for (int t = wave_id(); t < T; t += kPermWaves)
                topk_token<EPL>(logits, t, E, k, score, ids, w, s_ids);
            __syncthreads();
            permute_block(s_ids, T * k, E, offsets, sorted, inv, hdr);
            // the offsets written above are read back by this block only; the
            // barrier orders the global writes before those reads
            __syncthreads();
            build_schedule(offsets, E, T * k, tile_rows, max_tiles, active, tiles, split_cnt,
                           hdr);
        }
        return;
    }
    const int t = (blockIdx.x - 1) * kPermWaves + wave_id();   // one wavefront per token row
    if (t >= T) return;
    stage_x_row(x, act_bf16, H, t, x16, xsum, xe, hdr);
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
    const int grid = 1 + (a.T + kPermWaves - 1) / kPermWaves;
    const int epl = (d.n_experts + kWave - 1) / kWave;
#define FW_FRONT(N)                                                                            \
    case N:                                                                                    \
        if (small)                                                                             \
            decode_front_kernel<N, true><<<grid, kPermThreads, 0, s>>>(FW_FRONT_ARGS);         \
        else                                                                                   \
            decode_front_kernel<N, false><<<grid, kPermThreads, 0, s>>>(FW_FRONT_ARGS);        \
        break;
#define FW_FRONT_ARGS                                                                          \
    logits, a.T, d.n_experts, d.top_k, d.score, ids, w, offsets, sorted, inv, a.x,             \
        d.act_dtype == FW_BF16, d.hidden, kGemvTokens, a.L.max_tiles,                          \
        (int4 *)(a.ws + a.L.active), (int4 *)(a.ws + a.L.tiles), (_Float16 *)(a.ws + a.L.x16), \
        sums ? (float *)(a.ws + a.L.xsum) : nullptr, (int32_t *)(a.ws + a.L.xe),               \
        (int *)(a.ws + a.L.split_cnt), (WsHeader *)a.ws
    const bool small = (long long)a.T * d.top_k <= kSmallP;
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
#undef FW_FRONT_ARGS
#undef FW_FRONT
    return hipGetLastError();
}

}  // namespace fw
