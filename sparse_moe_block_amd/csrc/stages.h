// Device code shared by the stage kernels and the fused decode front end:
// wavefront reductions and the per-token top-k (route), the one-workgroup
// permutation, and the forward's schedule and activation staging.
#pragma once

#include "common.h"

namespace fw {

constexpr int kPrepThreads = 256;
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

// Wave-wide reductions on the DPP network (no LDS round trip): quad
// permutations, half-row and row mirrors leave every lane of a row with the
// row's result; row broadcasts 15 and 31 carry it into rows 1..3; lane 63
// holds the wave's result.  Fixed pattern, so sums are deterministic.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp<0xB1>(v));         // quad_perm [1,0,3,2]
    v = max(v, dpp<0x4E>(v));         // quad_perm [2,3,0,1]
    v = max(v, dpp<0x141>(v));        // row_half_mirror
    v = max(v, dpp<0x140>(v));        // row_mirror
    v = max(v, dpp<0x142, 0xA>(v));   // row_bcast:15 into rows 1, 3
    v = max(v, dpp<0x143, 0xC>(v));   // row_bcast:31 into rows 2, 3
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float fdpp_add(float v, uint32_t o) { return v + __uint_as_float(o); }
__device__ __forceinline__ float wave_sum_f32(float v) {
    v = fdpp_add(v, dpp<0xB1>(__float_as_uint(v)));
    v = fdpp_add(v, dpp<0x4E>(__float_as_uint(v)));
    v = fdpp_add(v, dpp<0x141>(__float_as_uint(v)));
    v = fdpp_add(v, dpp<0x140>(__float_as_uint(v)));
    // rows 1 and 3 add lane 15 / 47; rows 0 and 2 add nothing (the DPP keeps
    // their own value, so subtract-free: mask them out of the add instead)
    {
        const uint32_t o = dpp<0x142, 0xA>(__float_as_uint(v));
        const bool add = (__lane_id() >> 4) & 1;
        v = add ? v + __uint_as_float(o) : v;
    }
    {
        const uint32_t o = dpp<0x143, 0xC>(__float_as_uint(v));
        const bool add = (__lane_id() >> 5) & 1;
        v = add ? v + __uint_as_float(o) : v;
    }
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// Total order of logits as unsigned keys: larger logit -> larger key; -0 and
// +0 compare equal (both map to the key of +0), NaN maps below -inf.
__device__ __forceinline__ uint32_t logit_key(float l) {
    if (l != l) return 0u;
    const uint32_t u = __float_as_uint(l + 0.0f);   // -0 + 0 = +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// One wavefront per token.  Lane l holds the logits of experts l, l+64, ...
// as keys; each of k rounds takes the wave maximum of the untaken keys (DPP),
// then the lowest expert index holding it (one ballot per register), so the
// experts come out in descending logit order with ties to the lower index;
// lane j keeps slot j.  Renormalised weights: softmax -> exp(l_j - l_0) / sum
// over the slots (l_0 is the maximum); sigmoid -> s_j / sum s.
// Called by a whole wavefront for token t (wave-uniform); lds_ids, when set,
// also receives the token's ids (the fused decode front end).
template <int EPL>
__device__ __forceinline__ void topk_token(const float *__restrict__ logits, int t, int E, int k,
                                           int score, int32_t *__restrict__ ids,
                                           float *__restrict__ w, int32_t *lds_ids) {
    const int lane = threadIdx.x % kWave;
    uint32_t key[EPL];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        key[i] = e < E ? logit_key(logits[(size_t)t * E + e]) : 0u;
        if (e >= E) taken |= 1u << i;   // never selectable
    }
    int my_e = 0;
    float my_l = 0.f;
    for (int j = 0; j < k; ++j) {
        uint32_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (!((taken >> i) & 1u)) best = max(best, key[i]);
        const uint32_t m = wave_max_u32(best);
        int sel = 0;
#pragma unroll
        for (int i = EPL - 1; i >= 0; --i) {   // the lowest i with a match wins
            const unsigned long long b = __ballot(!((taken >> i) & 1u) && key[i] == m);
            if (b) sel = kWave * i + __builtin_ctzll(b);
        }
        if ((sel % kWave) == lane) taken |= 1u << (sel / kWave);
        if (lane == j) {
            my_e = sel;
            my_l = key_logit(m);
        }
    }
    const float l0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(my_l), 0));
    float s = 0.f;
    if (lane < k) s = score == FW_SOFTMAX_RENORM ? expf(my_l - l0) : 1.0f / (1.0f + expf(-my_l));
    const float sum = wave_sum_f32(s);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        w[(size_t)t * k + lane] = s / sum;
        if (lds_ids) lds_ids[t * k + lane] = my_e;
    }
}


// The one-workgroup stable counting sort (kPermThreads threads, all of which
// must call it).  ids may point to global memory or to LDS.
__device__ __forceinline__ void permute_block(const int32_t *ids, int P, int E,
                                              int32_t *__restrict__ offsets,
                                              int32_t *__restrict__ sorted,
                                              int32_t *__restrict__ inv,
                                              WsHeader *__restrict__ hdr) {
    __shared__ int cnt[kMaxExperts];
    __shared__ int cursor[kMaxExperts];
    __shared__ int wave_tot[kMaxExperts / kWave];
    __shared__ int wcnt[kPermWaves][kMaxExperts];
    __shared__ int n_valid;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

    for (int e = tid; e < kMaxExperts; e += kPermThreads) cnt[e] = 0;
    for (int i = tid; i < kPermWaves * kMaxExperts; i += kPermThreads) (&wcnt[0][0])[i] = 0;
    __syncthreads();

    bool bad = false;
    for (int q = tid; q < P; q += kPermThreads) {
        const int e = ids[q];
        if ((unsigned)e < (unsigned)E)
            atomicAdd(&cnt[e], 1);
        else
            bad = true;
    }
    if (bad) atomicOr(&hdr->status, FW_STATUS_BAD_EXPERT_ID);
    __syncthreads();

    // exclusive scan over E <= 512 counts: waves 0..7 scan 64 experts each
    if (tid < kMaxExperts) {
        const int v = tid < E ? cnt[tid] : 0;
        int incl = v;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        if (lane == kWave - 1) wave_tot[wave] = incl;
        cnt[tid] = incl - v;   // exclusive within the wave
    }
    __syncthreads();
    if (tid < kMaxExperts) {
        int base = 0;
        for (int w = 0; w < wave; ++w) base += wave_tot[w];
        const int ex = cnt[tid] + base;
        if (tid <= E) offsets[tid] = ex;   // offsets[E] = total valid
        if (tid == E) n_valid = ex;
        if (tid < E) cursor[tid] = ex;
    }
    if (E == kMaxExperts && tid == 0) {
        int tot = 0;
        for (int w = 0; w < kMaxExperts / kWave; ++w) tot += wave_tot[w];
        offsets[E] = tot;
        n_valid = tot;
    }
    __syncthreads();

    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    for (int c = 0; c * kPermThreads < P; ++c) {
        const int q = c * kPermThreads + tid;
        const int e = q < P ? ids[q] : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        unsigned long long peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 9; ++b) {   // E <= 512: 9 id bits
            const bool bit = valid && ((e >> b) & 1);
            const unsigned long long m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & lt_mask);
        const int tag = (c + 1) << 8;   // counts are <= 64 < 256
        if (valid && rank == 0) wcnt[wave][e] = tag | __popcll(peers);
        __syncthreads();
        int prefix = 0, total = 0;
        if (valid) {
            for (int w = 0; w < kPermWaves; ++w) {
                const int v = wcnt[w][e];
                const int n = (v & ~0xFF) == tag ? (v & 0xFF) : 0;
                if (w < wave) prefix += n;
                total += n;
            }
            const int pos = cursor[e] + prefix + rank;   // < offsets[e+1] <= P
            if ((unsigned)pos < (unsigned)P) {
                sorted[pos] = q;
                inv[q] = pos;
            }
        } else if (q < P) {
            inv[q] = -1;
        }
        __syncthreads();
        if (valid && prefix + rank == total - 1) cursor[e] += total;
        // the next chunk's LDS reads of cursor[] follow its first barrier
    }
    __syncthreads();
    for (int p = n_valid + tid; p < P; p += kPermThreads) sorted[p] = -1;
}


// Work estimate of a GEMM row tile of r rows, used to split the tile list
// among the XCDs (TileCost: a fixed part for an expert's first tile and for
// each later one, and a part per 32-row MFMA group).
__device__ __forceinline__ int gemm_tile_work(int r, bool first, TileCost c) {
    return (first ? c.first : c.rep) + c.group * ((r + 31) / 32);
}

// Block-0 part of the forward's staging: the active-expert list and the row
// tiles from expert_offsets, and the GEMV split-K arrival counters cleared.
// Thread tid owns experts 2*tid and 2*tid+1, so a block of 256 to 1024
// threads covers E <= 512; every thread of the block must call it.
// GEMM tiles (tile_rows >= 32) are also split among the 8 XCDs: contiguous
// ranges of about equal work (gemm_tile_work), each at most xcd_tile_cap
// tiles, in hdr->xcd_first.  Tiles are in expert order, so the tiles of an
// expert share an XCD's L2 unless a boundary falls inside them.
__device__ __forceinline__ void build_schedule(const int32_t *offsets, int E, int P,
                                               int tile_rows, int max_tiles,
                                               int4 *__restrict__ active, int4 *__restrict__ tiles,
                                               int *__restrict__ split_cnt,
                                               WsHeader *__restrict__ hdr,
                                               TileCost cost = TileCost{1, 1, 0}) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const bool balance = tile_rows >= 32;
    // the GEMV's split-K arrival counters start every call at zero
    for (int i = tid; i < kSplitTiles; i += blockDim.x) split_cnt[i] = 0;
    // one entry per wave of a block of up to 1024 threads: threads from 256
    // on own experts >= 512 >= E, so they contribute zeros
    __shared__ int wsum_a[1024 / kWave], wsum_t[1024 / kWave], wsum_w[1024 / kWave];
    __shared__ int s_first[8];   // raw XCD boundaries: the tile holding 1/8 .. 7/8 of the work
    // each thread owns experts 2*tid and 2*tid+1
    int beg[2], cnt[2], na = 0, nt = 0, nw = 0;
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
            if (balance) {
                const int full = cnt[i] / tile_rows, rem = cnt[i] % tile_rows;
                if (full) nw += gemm_tile_work(tile_rows, true, cost) +
                                (full - 1) * gemm_tile_work(tile_rows, false, cost);
                if (rem) nw += gemm_tile_work(rem, full == 0, cost);
            }
        }
    }
    if (bad) atomicOr(&hdr->status, FW_STATUS_BAD_OFFSETS);
    if (tid < 8) s_first[tid] = 0x7FFFFFFF;
    int ia = na, it = nt, iw = nw;   // inclusive scans
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int oa = __shfl_up(ia, off), ot = __shfl_up(it, off), ow = __shfl_up(iw, off);
        if (lane >= off) {
            ia += oa;
            it += ot;
            iw += ow;
        }
    }
    if (lane == kWave - 1) {
        wsum_a[wave] = ia;
        wsum_t[wave] = it;
        wsum_w[wave] = iw;
    }
    __syncthreads();
    int ba = 0, bt = 0, bw = 0, total_t = 0, total_w = 0;
    for (int w = 0; w < (int)blockDim.x / kWave; ++w) {
        if (w < wave) {
            ba += wsum_a[w];
            bt += wsum_t[w];
            bw += wsum_w[w];
        }
        total_t += wsum_t[w];
        total_w += wsum_w[w];
    }
    int pa = ba + ia - na, pt = bt + it - nt, pw = bw + iw - nw;   // exclusive positions
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (cnt[i] > 0) {
            active[pa++] = int4{2 * tid + i, beg[i], cnt[i], 0};
            // bounded: overlapping (invalid) offsets can claim more
            for (int m = 0; m < cnt[i] && pt < max_tiles; m += tile_rows) {
                const int r = min(tile_rows, cnt[i] - m);
                tiles[pt] = int4{2 * tid + i, beg[i] + m, r, 0};
                if (balance) {
                    // the tile holding the point x/8 of the work starts XCD
                    // x's range if less than half of it lies before the point
                    const int w = gemm_tile_work(r, m == 0, cost);
                    for (int x = 1; x < 8; ++x) {
                        const int64_t at = (int64_t)x * total_w - 8 * (int64_t)pw;
                        if (at >= 0 && at < 8 * (int64_t)w) s_first[x] = at < 4 * w ? pt : pt + 1;
                    }
                    pw += w;
                }
                ++pt;
            }
        }
    }
    const int n_tiles = min(total_t, max_tiles);
    if (tid == kPrepThreads - 1) {
        hdr->n_active = ba + ia;
        hdr->n_tiles = n_tiles;
    }
    if (balance) {
        __syncthreads();
        if (tid == 0) {
            // capped ranges: none longer than cap, and each leaves the XCDs
            // after it no more than they have room for
            const int cap = xcd_tile_cap(P, E, tile_rows, max_tiles);
            const int n = min(n_tiles, 8 * cap);
            int f = 0;
            hdr->xcd_first[0] = 0;
            for (int x = 1; x < 8; ++x) {
                const int lo = max(f, n - (8 - x) * cap), hi = min(f + cap, n);
                f = min(max(s_first[x], lo), hi);
                hdr->xcd_first[x] = f;
            }
            hdr->xcd_first[8] = n;
        }
    }
}

// The 32 values of block b of token row t as fp32 (bf16 widened exactly).
__device__ __forceinline__ void load_x_block(const void *__restrict__ x, int act_bf16, int H,
                                             int t, int b, float *v) {
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
}

// One wavefront stages token row t (called by the whole wavefront, t uniform):
// the row's largest magnitude sets its exponent e (x * 2^e has its largest
// magnitude in [2^(kXExp-1), 2^kXExp); e = 0 for an all-zero row), written to
// xe[t]; then every 32-element block is stored as fp16 x * 2^e in the pair
// order both kernel families consume (see decode_pairs; pairs j = 1, 3 at
// 1/16), with, when xsum is set, the block's sum of the stored values (the
// min term of a Q4_K GEMV).  A non-finite value sets FW_STATUS_RANGE.
__device__ __forceinline__ void stage_x_row(const void *__restrict__ x, int act_bf16, int H,
                                            int t, _Float16 *__restrict__ x16,
                                            float *__restrict__ xsum, int32_t *__restrict__ xe,
                                            WsHeader *__restrict__ hdr) {
    const int lane = threadIdx.x % kWave, nb = H / 32;
    // |v| as fp32 bits orders like |v| (NaN above +inf)
    uint32_t m = 0;
    for (int b = lane; b < nb; b += kWave) {
        float v[32];
        load_x_block(x, act_bf16, H, t, b, v);
#pragma unroll
        for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    }
    m = wave_max_u32(m);
    int e = 0;
    if (m >= 0x7F800000u) {
        if (lane == 0) atomicOr(&hdr->status, FW_STATUS_RANGE);
    } else if (m != 0) {
        // amax = f * 2^E, f in [0.5, 1): amax * 2^(kXExp - E) in [2^(kXExp-1), 2^kXExp)
        e = kXExp - __builtin_amdgcn_frexp_expf(__uint_as_float(m));
    }
    if (lane == 0) xe[t] = e;
    for (int b = lane; b < nb; b += kWave) {
        float v[32];
        load_x_block(x, act_bf16, H, t, b, v);
        uint32_t o[16];
#pragma unroll
        for (int pi = 0; pi < 16; ++pi) {
            const int mm = pi >> 2, j = pi & 3;
            const int e0 = (j & 1 ? 16 : 0) + 4 * mm + (j >> 1);
            const int es = (j & 1) ? e - 4 : e;
            o[pi] = __builtin_bit_cast(uint32_t,
                                       h2{(_Float16)__builtin_amdgcn_ldexpf(v[e0], es),
                                          (_Float16)__builtin_amdgcn_ldexpf(v[e0 + 2], es)});
        }
        uint4 *dst = (uint4 *)(x16 + (size_t)t * H + 32 * b);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            dst[q] = uint4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
        if (xsum) {
            // the block's sum of the stored fp16 values (pairs j = 1, 3 back at
            // full scale), in pair order
            float sum = 0.f;
#pragma unroll
            for (int pi = 0; pi < 16; ++pi) {
                const h2 hv = as_h2(o[pi]);
                const float sc = (pi & 1) ? 16.0f : 1.0f;
                sum += sc * (float)hv[0];
                sum += sc * (float)hv[1];
            }
            xsum[(size_t)t * nb + b] = sum;
        }
    }
}

}  // namespace fw
