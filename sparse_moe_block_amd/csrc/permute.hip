// Token -> expert grouping: a stable counting sort of the T*k (token, slot)
// pairs by expert, in one workgroup, all on the device (the pages' runtime has
// host synchronisation points here -- Flyweight 0.2.0 "Current limitations").
//
// 1. LDS histogram of the expert ids (integer atomics: order-free).
// 2. Exclusive scan of the counts -> expert_offsets and per-expert cursors.
// 3. Chunks of 1024 pairs in pair order.  Inside a wave, the lanes holding the
//    same expert find each other with ballots over the id bits; a lane's rank
//    among them plus the counts of the same expert in lower waves of the chunk
//    (published in LDS, tagged with the chunk number) plus the expert's cursor
//    is the pair's final position.  The position is therefore the stable one
//    (ascending pair id within an expert) whatever the scheduling.
//
// Above a few thousand pairs one workgroup walking the chunks in turn is the
// bottleneck (16 chunks of a 2048-token, top-8 batch: about 35 us), so large
// batches run the same sort as three kernels, one chunk per workgroup:
//   count:   per-chunk LDS histograms -> cnt[e][b];
//   scan:    one workgroup per expert turns its row into the exclusive prefix
//            over chunks and appends the expert's total;
//   scatter: every chunk workgroup scans the totals into expert_offsets (chunk
//            0 writes them) and places its pairs at offset + prefix + the
//            in-chunk rank of step 3.  Same positions as the one-workgroup sort.
// Up to kPermFoldChunks chunks the scan is folded into the scatter: each
// chunk workgroup sums the raw counts of the chunks before it itself (a few
// KB of reads), which saves a launch.
#include "common.h"
#include "stages.h"

namespace fw {
namespace {

constexpr int kThreads = 1024;
constexpr int kPermFoldChunks = 64;
constexpr int kWaves = kThreads / kWave;

__global__ __launch_bounds__(kThreads) void permute_kernel(
    const int32_t *__restrict__ ids, int P, int E, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted, int32_t *__restrict__ inv, WsHeader *__restrict__ hdr) {
    permute_block(ids, P, E, offsets, sorted, inv, hdr);
}

// Exclusive scan of per-expert values v (threads tid < kMaxExperts hold one
// each, zero past E) over a 1024-thread workgroup; returns the exclusive prefix
// to threads tid < kMaxExperts and writes the sum of all to *total.
__device__ __forceinline__ int expert_scan(int v, int *wave_tot, int *total) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    int incl = v;
    if (tid < kMaxExperts) {
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        if (lane == kWave - 1) wave_tot[wave] = incl;
    }
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kMaxExperts / kWave; ++w) {
        if (w < wave) base += wave_tot[w];
        tot += wave_tot[w];
    }
    if (tid == 0) *total = tot;
    return base + incl - v;
}

__global__ __launch_bounds__(kThreads) void perm_count_kernel(
    const int32_t *__restrict__ ids, int P, int E, int nb, int32_t *__restrict__ cnt_g,
    WsHeader *__restrict__ hdr) {
    __shared__ int cnt[kMaxExperts];
    const int tid = threadIdx.x, b = blockIdx.x;
    for (int e = tid; e < E; e += kThreads) cnt[e] = 0;
    __syncthreads();
    const int q = b * kPermChunk + tid;
    if (q < P) {
        const int e = ids[q];
        if ((unsigned)e < (unsigned)E)
            atomicAdd(&cnt[e], 1);
        else
            atomicOr(&hdr->status, FW_STATUS_BAD_EXPERT_ID);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) cnt_g[(size_t)e * (nb + 1) + b] = cnt[e];
}

// One workgroup per expert: exclusive prefix of its per-chunk counts, in place,
// and the expert's total in column nb.
__global__ __launch_bounds__(256) void perm_scan_kernel(int nb, int32_t *__restrict__ cnt_g) {
    __shared__ int wt[4];
    int32_t *row = cnt_g + (size_t)blockIdx.x * (nb + 1);
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int per = (nb + 255) / 256, b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
    int sum = 0;
    for (int b = b0; b < b1; ++b) sum += row[b];
    int incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wt[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wt[w];
    int run = base + incl - sum;
    for (int b = b0; b < b1; ++b) {
        const int v = row[b];
        row[b] = run;
        run += v;
    }
    if (tid == 255) row[nb] = base + incl;
}

__global__ __launch_bounds__(kThreads) void perm_scatter_kernel(
    const int32_t *__restrict__ ids, int P, int E, int nb, const int32_t *__restrict__ cnt_g,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted, int32_t *__restrict__ inv,
    int fold) {
    __shared__ int cursor[kMaxExperts];
    __shared__ int wave_tot[kMaxExperts / kWave];
    __shared__ int wcnt[kWaves][kMaxExperts];
    __shared__ int n_valid;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, b = blockIdx.x;
    for (int i = tid; i < kWaves * kMaxExperts; i += kThreads) (&wcnt[0][0])[i] = 0;
    // this expert's total and its count in the chunks before this one: raw
    // counts summed here (fold) or the scan kernel's prefix and total
    int v = 0, before = 0;
    if (tid < E) {
        const int32_t *row = cnt_g + (size_t)tid * (nb + 1);
        if (fold) {
            for (int c = 0; c < nb; ++c) {
                const int n = row[c];
                v += n;
                before += c < b ? n : 0;
            }
        } else {
            v = row[nb];
            before = row[b];
        }
    }
    const int ex = expert_scan(v, wave_tot, &n_valid);
    if (tid < E) cursor[tid] = ex + before;
    if (b == 0 && tid < E) offsets[tid] = ex;
    __syncthreads();
    if (b == 0 && tid == 0) offsets[E] = n_valid;

    // this chunk's pairs: rank among the same expert's pairs of the chunk
    const int q = b * kPermChunk + tid;
    const int e = q < P ? ids[q] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {   // E <= 512: 9 id bits
        const bool on = valid && ((e >> bit) & 1);
        const unsigned long long m = __ballot(on);
        peers &= on ? m : ~m;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    if (valid && rank == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
        int prefix = 0;
        for (int w = 0; w < wave; ++w) prefix += wcnt[w][e];
        const int pos = cursor[e] + prefix + rank;
        if ((unsigned)pos < (unsigned)P) {
            sorted[pos] = q;
            inv[q] = pos;
        }
    } else if (q < P) {
        inv[q] = -1;
    }
    for (int p = n_valid + q; p < P; p += nb * kPermChunk) sorted[p] = -1;
}

__global__ void clear_status_kernel(WsHeader *hdr) {
    if (threadIdx.x == 0) hdr->status = 0;
}

__global__ void copy_status_kernel(const WsHeader *hdr, int32_t *status) {
    if (threadIdx.x == 0) *status = hdr->status;
}

}  // namespace

hipError_t launch_permute(const fw_moe_desc &d, int T, const int32_t *ids, int32_t *offsets,
                          int32_t *sorted, int32_t *inv, WsHeader *hdr, int32_t *perm,
                          hipStream_t s) {
    const int P = T * d.top_k, E = d.n_experts;
    if (P <= kPermOneBlockMaxP) {
        permute_kernel<<<1, kThreads, 0, s>>>(ids, P, E, offsets, sorted, inv, hdr);
        return hipGetLastError();
    }
    const int nb = perm_blocks(P);
    const int fold = nb <= kPermFoldChunks;
    perm_count_kernel<<<nb, kThreads, 0, s>>>(ids, P, E, nb, perm, hdr);
    if (!fold) perm_scan_kernel<<<E, 256, 0, s>>>(nb, perm);
    perm_scatter_kernel<<<nb, kThreads, 0, s>>>(ids, P, E, nb, perm, offsets, sorted, inv, fold);
    return hipGetLastError();
}

hipError_t launch_clear_status(WsHeader *hdr, hipStream_t s) {
    clear_status_kernel<<<1, 64, 0, s>>>(hdr);
    return hipGetLastError();
}

hipError_t launch_copy_status(const WsHeader *hdr, int32_t *status, hipStream_t s) {
    copy_status_kernel<<<1, 64, 0, s>>>(hdr, status);
    return hipGetLastError();
}

}  // namespace fw
