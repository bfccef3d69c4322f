// Forward with MXFP8 expert activations on MXFP4 experts: the staging of x as
// MXFP8, and the grouped expert GEMMs on gfx950's block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 activations x E2M1 weights, one
// E8M0 scale per operand row and 32-element block, fp32 accumulation).  The
// MX formats with group 32 (MXFP4 experts, the MXFP8 alternative) are vOOM's
// (lossy artifact notes); the block quantisation is the OCP MX one: per 32
// values the scale 2^(floor(log2 amax) - 8) and E4M3 elements, nearest-even,
// clamped at 448.
//
// The weights reach the matrix cores as stored: no dequantisation at all.
// Per workgroup a tile of up to 160 rows (five 32-row groups) of one
// expert's pairs times 256 weight rows; eight wavefronts (two per SIMD),
// wavefront w taking row half w / 4 and weight quarter w % 4: of a tile's
// MI row groups the first half takes two (three when MI = 5), the second the
// rest, each against 64 weight rows (two 32-column groups), so each SIMD runs
// 2 MI MFMAs per 64-k slice.  (Four wavefronts of 128 rows each left one
// wavefront per SIMD, nothing to run while it waited at the step's
// rendezvous.)  Each tile streams its expert's weights, so an expert of
// 129-160 rows is one tile rather than a full one plus a one-group one.  K
// advances 256 per step (four slices); a step's activation codes (160 x 256
// bytes) and scales, and
// its weight codes (256 x 128 bytes) and scales move HBM/L2 -> LDS by DMA
// into one of two buffer sets while the other is used.
//
// Operand layout of the MFMA (per lane l, i = l % 32, h = l / 32; within a
// 64-k slice): the E4M3 operand's 32 bytes are k 16h .. 16h + 15 then
// 32 + 16h .. 32 + 16h + 15 of row i; the E2M1 operand's 32 nibbles are k
// 32h .. 32h + 31 of column i, low nibble first; each operand's scale byte
// from lane l covers row (column) i and k-block h of the slice.  The scale
// register carries four bytes (op_sel picks one): a lane keeps the step's
// blocks h, 2 + h, 4 + h, 6 + h, byte S for slice S.
#include <math.h>

#include "common.h"
#include "stages.h"

namespace fw {
namespace {

constexpr int MBM = 160;         // token rows per tile
constexpr int MBN = 256;         // weight rows per tile
constexpr int MKS = 256;         // k per step
constexpr int MNW = 8;           // wavefronts per workgroup (two per SIMD)
constexpr int MThreads = 64 * MNW;
constexpr int kAChunks = MBM * MKS / 16;   // 16-byte chunks of a step's activation codes: 2560
constexpr int kBChunks = MBN * MKS / 32;   // of its weight codes: 2048
static_assert(MBM == 160 && 2 * MBM <= MThreads, "tile shape");

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// ---- MXFP8 quantisation ----------------------------------------------------
// E8M0 exponent of a block whose largest magnitude is amax (> 0, finite):
// floor(log2 amax) - 8, clamped to -127 .. 127.
__device__ __forceinline__ int mx8_exp(float amax) {
    const int e = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;
    return min(max(e, -127), 127);
}
// E4M3 code of v * 2^-e: exact scaling, clamp to +-448, nearest-even (the
// conversion returns NaN above 464, hence the clamp).
__device__ __forceinline__ uint32_t mx8_code(float v, int e) {
    const float y = fminf(fmaxf(__builtin_amdgcn_ldexpf(v, -e), -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFFu;
}

// One wavefront stages token row t as MXFP8: each lane quantises whole
// 32-element blocks (codes in k order to x8, the E8M0 byte to xs).  A
// non-finite value sets FW_STATUS_RANGE.
__device__ __forceinline__ void stage_x_row_mx8(const void *__restrict__ x, int act_bf16, int H,
                                                int t, uint8_t *__restrict__ x8,
                                                uint8_t *__restrict__ xs,
                                                WsHeader *__restrict__ hdr) {
    const int lane = threadIdx.x % kWave, nb = H / 32;
    bool bad = false;
    for (int b = lane; b < nb; b += kWave) {
        float v[32];
        load_x_block(x, act_bf16, H, t, b, v);
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
        bad |= m >= 0x7F800000u;
        const int e = m == 0 ? -127 : mx8_exp(__uint_as_float(m));
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) w |= mx8_code(v[4 * q + j], e) << (8 * j);
            o[q] = w;
        }
        uint4 *dst = (uint4 *)(x8 + (size_t)t * H + 32 * b);
        dst[0] = uint4{o[0], o[1], o[2], o[3]};
        dst[1] = uint4{o[4], o[5], o[6], o[7]};
        xs[(size_t)t * nb + b] = (uint8_t)(m == 0 ? 0 : e + 127);
    }
    if (bad) atomicOr(&hdr->status, FW_STATUS_RANGE);
}

// Block 0: the schedule (active experts, 160-row tiles); the other blocks:
// one wavefront per token row, staged as MXFP8.
__global__ __launch_bounds__(kPrepThreads) void prepare_mx8_kernel(
    const int32_t *__restrict__ offsets, int E, int P, const void *__restrict__ x, int act_bf16,
    int H, int T, int max_tiles, int4 *__restrict__ active, int4 *__restrict__ tiles,
    uint8_t *__restrict__ x8, uint8_t *__restrict__ xs, int *__restrict__ split_cnt,
    WsHeader *__restrict__ hdr) {
    if (blockIdx.x == 0) {
        build_schedule(offsets, E, P, MBM, max_tiles, active, tiles, split_cnt, hdr,
                       kCostMx8);
        return;
    }
    const int t = (blockIdx.x - 1) * (kPrepThreads / kWave) + wave_id();
    if (t >= T) return;
    stage_x_row_mx8(x, act_bf16, H, t, x8, xs, hdr);
}

// ---- the block-scaled grouped GEMM -----------------------------------------
// LDS weight row Rl of the tile:
//   gate/up: Rl < 128: gate feature 128 ct + Rl, else up feature 128 ct +
//            Rl - 128; weight quarter q reads rows 32 q + n (gate, column
//            group 0) and 128 + 32 q + n (up, column group 1), so a lane holds
//            gate and up of the same features, and the quarter's 32 features
//            are one 32-element block of h;
//   down:    output row 256 ct + Rl; weight quarter q reads 64 q + 32 cg + n.
template <bool GU> __device__ __forceinline__ int mx_wrow(int q, int cg, int n) {
    return GU ? 128 * cg + 32 * q + n : 64 * q + 32 * cg + n;
}

// The four scale bytes a lane of half h uses in one step: blocks h, 2 + h,
// 4 + h, 6 + h of the row's eight (byte S for slice S).
__device__ __forceinline__ uint32_t mx_scale_word(uint2 s8, int h) {
    return __builtin_amdgcn_perm(s8.y, s8.x, h ? 0x07050301u : 0x06040200u);
}

// One (row tile, column tile) of one expert (or of the shared expert).
//  GU:  A = x8 rows (routed: the tokens of the sorted pairs); weights = 128
//       gate + 128 up features; writes h = MXFP8(SiLU(g) * u) (codes to h8,
//       one E8M0 byte per row and 32 features to hsc), row stride ldh;
//  !GU: A = h8 rows (stride K); weights = 256 outputs; writes y (fp32).
template <bool GU>
__global__ __launch_bounds__(MThreads, 1) void gemm_mx_kernel(
    const uint8_t *__restrict__ wa, const uint8_t *__restrict__ wb,
    const int4 *__restrict__ tiles, WsHeader *__restrict__ hdr,
    const int32_t *__restrict__ sorted, const uint8_t *__restrict__ a8,
    const uint8_t *__restrict__ asc, uint8_t *__restrict__ h8, uint8_t *__restrict__ hsc,
    float *__restrict__ yout, int K, int N, int k, int P, int col_tiles, int n_row_tiles_max,
    int shared, int shared_rows, size_t sreg) {
    // two buffer sets, each its own array: the compiler tells a pending DMA
    // into one from reads of the other only when they are distinct objects
    __shared__ uint4 A0[kAChunks], A1[kAChunks];
    __shared__ uint4 B0[kBChunks], B1[kBChunks];
    // 8 scale bytes per row and step (dwords past 2 MBM: padding that the
    // scale DMA of the remaining threads writes, so that every thread issues it)
    __shared__ uint32_t AS0[MThreads], AS1[MThreads];
    __shared__ uint32_t BS0[MBN * 2], BS1[MBN * 2];
    auto Abuf = [&](int buf) { return buf ? A1 : A0; };
    auto Bbuf = [&](int buf) { return buf ? B1 : B0; };
    auto ASbuf = [&](int buf) { return buf ? AS1 : AS0; };
    auto BSbuf = [&](int buf) { return buf ? BS1 : BS0; };
    // XCD-aware order (the tiles of one expert are consecutive)
    int ct;
    const int rt = xcd_row_tile(hdr, col_tiles, n_row_tiles_max, shared,
                                (shared_rows + MBM - 1) / MBM, ct);
    if (rt < 0) return;
    int expert = 0, rb = 0, rows = 0;
    if (shared) {
        rb = rt * MBM;
        rows = min(MBM, shared_rows - rb);
    } else {
        const int4 tl = ld_const(tiles + rt);   // (expert, first row, rows)
        expert = tl.x;
        rb = tl.y;
        rows = tl.z;
    }
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int n = lane & 31, g = lane >> 5;
    const int rh = wave / 4, wq = wave % 4;   // the wavefront's row half and weight quarter
    // the activation row (token row, or h row) of tile row r
    auto src_row = [&](int r) {
        r = min(r, rows - 1);
        if (GU && !shared) {
            const int q = sorted[rb + r];
            return (unsigned)q < (unsigned)P ? q / k : 0;
        }
        return rb + r;
    };
    if (GU && !shared && tid < rows && (unsigned)sorted[rb + tid] >= (unsigned)P)
        atomicOr(&hdr->status, FW_STATUS_BAD_PAIR);
    // DMA slots: instruction i of thread tid fills LDS slot i * 512 + tid.
    // activation codes: slot s is position s % 16 of tile row s / 16 and holds
    // its chunk (s % 16) ^ (row % 16) (so that the 32 lanes reading one chunk
    // of 32 rows hit distinct banks); instruction i covers row group i
    uint32_t aoff[MBM / 32];
#pragma unroll
    for (int i = 0; i < MBM / 32; ++i) {
        const int s = i * MThreads + tid, r = s / 16, c = (s % 16) ^ (r % 16);
        aoff[i] = (uint32_t)src_row(r) * (uint32_t)K + 16u * c;
    }
    // activation scales: slot tid (< 2 MBM) is dword tid % 2 of row tid / 2's
    // 8 bytes; threads 2 MBM.. repeat those of threads 0.. into the padding
    const uint32_t asoff = (uint32_t)src_row((tid % (2 * MBM)) / 2) * (uint32_t)(K / 32) +
                           4u * (tid % 2);
    // weight rows: LDS row Rl is matrix row wrow(Rl) of the expert
    auto wrow = [&](int Rl) {
        if (GU) return ct * 128 + (Rl & 127);   // the gate or the up matrix's row
        return ct * 256 + Rl;
    };
    const uint8_t *gbase = wa + (size_t)expert * N * (K / 2);
    const uint8_t *ubase = (GU ? wb : wa) + (size_t)expert * N * (K / 2);
    const uint8_t *gsc = wa + sreg + (size_t)expert * N * (K / 32);
    const uint8_t *usc = (GU ? wb : wa) + sreg + (size_t)expert * N * (K / 32);
    // weight codes: slot s is position s % 8 of LDS row s / 8 and holds its
    // chunk (s % 8) ^ (row / 2 % 8); rows 128 .. 255 of a gate/up tile are the
    // up matrix's (instructions 2 and 3)
    uint32_t boff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s = i * MThreads + tid, Rl = s / 8, c = (s % 8) ^ ((Rl / 2) % 8);
        boff[i] = (uint32_t)wrow(Rl) * (uint32_t)(K / 2) + 16u * c;
    }
    // weight scales: slot tid is dword tid % 2 of row tid / 2 (rows 128 ..
    // 255 of a gate/up tile: the up matrix's, threads 256 ..)
    const uint32_t bsoff = (uint32_t)wrow(tid / 2) * (uint32_t)(K / 32) + 4u * (tid % 2);
    // The main loop for a tile of MI 32-row groups (the groups that hold rows:
    // their DMA only) of which this wavefront's row half holds MW (0 .. 3:
    // its fragments and MFMAs).  Both are template parameters so that the
    // loop body has no branch: the compiler would otherwise sink a step's
    // MFMAs past the DMA wait at its end.
    auto run = [&]<int MI, int MW>() __attribute__((always_inline)) {
    auto dma = [&](int buf, int st, int part) {
        const uint32_t ka = (uint32_t)st * MKS, kb = (uint32_t)st * (MKS / 2),
                       ks = (uint32_t)st * (MKS / 32);
        if (part == 0) {
#pragma unroll
            for (int i = 0; i < MI; ++i)   // rows 32 i .. 32 i + 31
                __builtin_amdgcn_global_load_lds(
                    a8 + (aoff[i] + ka), (lds_void *)(&Abuf(buf)[i * MThreads + 64 * wave]), 16, 0,
                    0);
            __builtin_amdgcn_global_load_lds(asc + (asoff + ks),
                                             (lds_void *)(&ASbuf(buf)[64 * wave]), 4, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_global_load_lds((GU && i >= 2 ? ubase : gbase) + (boff[i] + kb),
                                                 (lds_void *)(&Bbuf(buf)[i * MThreads + 64 * wave]),
                                                 16, 0, 0);
            __builtin_amdgcn_global_load_lds((GU && wave >= 4 ? usc : gsc) + (bsoff + ks),
                                             (lds_void *)(&BSbuf(buf)[64 * wave]), 4, 0, 0);
        }
    };
    // everything issued so far has landed and every wavefront is here
    auto sync = [&]() {
        __builtin_amdgcn_s_waitcnt(7 << 4);   // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    constexpr int MA = MW > 0 ? MW : 1;   // array extent (a row half may hold no rows)
    f16v acc[MA][2];
#pragma unroll
    for (int i = 0; i < MA; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int steps = K / MKS;
    const int wr[2] = {mx_wrow<GU>(wq, 0, n), mx_wrow<GU>(wq, 1, n)};
    constexpr int kHalf0 = MI > 4 ? 3 : 2;   // row groups of the first row half
    const int r0 = 32 * kHalf0 * rh + n;   // the lane's first tile row

    // one step from buffer set `buf`; pf(S) issues the next step's DMA after
    // slice S's MFMAs
    auto step = [&](int buf, auto &&pf) {
        uint32_t sa[MA], sb[2];
#pragma unroll
        for (int mi = 0; mi < MW; ++mi) {
            const int r = r0 + 32 * mi;
            sa[mi] = mx_scale_word(*(const uint2 *)&ASbuf(buf)[2 * r], g);
        }
#pragma unroll
        for (int cg = 0; cg < 2; ++cg)
            sb[cg] = mx_scale_word(*(const uint2 *)&BSbuf(buf)[2 * wr[cg]], g);
        v8i a[2][MA], b[2][2];
        // slice S's fragments: row r0 + 32 mi, chunks 4 S + g and 4 S + 2 + g;
        // weight row wr[cg], chunk 2 S + g
        auto load = [&](int X, int S) {
#pragma unroll
            for (int mi = 0; mi < MW; ++mi) {
                const int r = r0 + 32 * mi, x = r % 16;
                const uint4 lo = Abuf(buf)[16 * r + ((4 * S + g) ^ x)];
                const uint4 hi = Abuf(buf)[16 * r + ((4 * S + 2 + g) ^ x)];
                a[X][mi] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                               (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
            if constexpr (MW > 0) {
#pragma unroll
                for (int cg = 0; cg < 2; ++cg) {
                    const int Rl = wr[cg];
                    const uint4 q = Bbuf(buf)[8 * Rl + ((2 * S + g) ^ ((Rl / 2) % 8))];
                    b[X][cg] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
                }
            }
        };
        load(0, 0);
#define FW_MX_SLICE(S)                                                                       \
    {                                                                                        \
        constexpr int X = (S) & 1;                                                           \
        if constexpr ((S) < 3) load(X ^ 1, (S) + 1);                                         \
        _Pragma("unroll") for (int cg = 0; cg < 2; ++cg)                                     \
            _Pragma("unroll") for (int mi = 0; mi < MW; ++mi)                                \
                acc[mi][cg] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(               \
                    a[X][mi], b[X][cg], acc[mi][cg], 0, 4, (S), (int)sa[mi], (S),            \
                    (int)sb[cg]);                                                            \
        pf(S);                                                                               \
        __builtin_amdgcn_sched_barrier(0);                                                   \
    }
        FW_MX_SLICE(0)
        FW_MX_SLICE(1)
        FW_MX_SLICE(2)
        FW_MX_SLICE(3)
#undef FW_MX_SLICE
    };
    // Step st uses buffer set st % 2 and loads step st + 1 into the other,
    // which every wavefront finished reading before the sync that ended step
    // st - 1.  Steps go in pairs (the loop body has no branch around its
    // DMA); after the last pair the prefetch repeats step steps - 1's
    // addresses, which is the step an odd count (K = 768: 3 steps) still has
    // to run, from buffer set 0.  No DMA reaches past step steps - 1.
    dma(0, 0, 0);
    dma(0, 0, 1);
    sync();
    int st = 0;
    for (; st + 1 < steps; st += 2) {
        step(0, [&](int S) { if (S < 2) dma(1, st + 1, S); });
        sync();
        const int nx = min(st + 2, steps - 1);
        step(1, [&](int S) { if (S < 2) dma(0, nx, S); });
        sync();
    }
    if (st < steps) step(0, [](int) {});

    // ---- epilogue: acc[mi][cg][v] is tile row r0 - n + 32 mi + 8 (v / 4) +
    // 4 g + v % 4, LDS weight row wr[cg] ----
    bool range = false;
    if constexpr (GU) {
        // features 128 ct + 32 wq + n: one 32-element block of h per row,
        // spread over the 32 lanes of a half-wavefront
        const int f0 = 128 * ct + 32 * wq;
#pragma unroll
        for (int mi = 0; mi < MW; ++mi)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = r0 - n + 32 * mi + 8 * (v >> 2) + 4 * g + (v & 3);
                const float gv = acc[mi][0][v], up = acc[mi][1][v];
                const float av = gv / (1.0f + __expf(-gv)) * up;
                uint32_t m = __float_as_uint(av) & 0x7FFFFFFFu;
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 32));
                if (row < rows) {
                    range |= m >= 0x7F800000u;
                    const int e = m == 0 ? -127 : mx8_exp(__uint_as_float(m));
                    const size_t hr = (size_t)(rb + row);
                    h8[hr * N + f0 + n] = (uint8_t)mx8_code(av, e);
                    if (n == 0) hsc[hr * (N / 32) + f0 / 32] = (uint8_t)(m == 0 ? 0 : e + 127);
                }
            }
    } else {
        float *yrow = yout + (size_t)ct * 256 + 64 * wq + n;
#pragma unroll
        for (int mi = 0; mi < MW; ++mi)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = r0 - n + 32 * mi + 8 * (v >> 2) + 4 * g + (v & 3);
                if (row < rows) {
#pragma unroll
                    for (int cg = 0; cg < 2; ++cg)
                        yrow[(size_t)(rb + row) * N + 32 * cg] = acc[mi][cg][v];
                }
            }
    }
    if (range) atomicOr(&hdr->status, FW_STATUS_RANGE);
    };
    // the tile's row groups, and the share of this wavefront's row half
    auto go = [&]<int MI>() __attribute__((always_inline)) {
        constexpr int H0 = MI > 4 ? 3 : 2;
        if (rh == 0) run.template operator()<MI, (MI < H0 ? MI : H0)>();
        else run.template operator()<MI, (MI > H0 ? MI - H0 : 0)>();
    };
    const int mi = (rows + 31) / 32;
    if (mi > 4) go.template operator()<5>();
    else if (mi > 3) go.template operator()<4>();
    else if (mi > 2) go.template operator()<3>();
    else if (mi > 1) go.template operator()<2>();
    else go.template operator()<1>();
}

// The MXFP8 areas inside the fp16 staging areas of the workspace: x8 [T][H]
// then its scales [T][H/32]; h8 [P][F] then [T][Fs], then their scales.
struct Mx8Areas {
    uint8_t *x8, *xs, *h8, *hs;
    size_t hrows;   // bytes of h8: P F + T Fs
};
Mx8Areas mx8_areas(const FwdArgs &a) {
    Mx8Areas m;
    m.x8 = (uint8_t *)(a.ws + a.L.x16);
    m.xs = m.x8 + (size_t)a.T * a.d.hidden;
    m.h8 = (uint8_t *)(a.ws + a.L.h);
    m.hrows = (size_t)a.P * a.d.ffn + (size_t)a.T * a.d.shared_ffn;
    m.hs = m.h8 + m.hrows;
    return m;
}

template <bool GU>
void launch_mx(const FwdArgs &a, const uint8_t *wa, const uint8_t *wb, const uint8_t *a8,
               const uint8_t *asc, uint8_t *h8, uint8_t *hsc, float *yout, int K, int N,
               int shared, hipStream_t s) {
    const int col_tiles = GU ? N / 128 : N / 256;
    const int row_tiles = shared ? (a.T + MBM - 1) / MBM
                                 : gemm_row_tiles(a.P, a.d.n_experts, MBM, a.L.max_tiles);
    const int nblk = (row_tiles + 7) / 8 * 8 * col_tiles;   // eight XCDs x whole row tiles
    gemm_mx_kernel<GU><<<nblk, MThreads, 0, s>>>(
        wa, wb, (const int4 *)(a.ws + a.L.tiles), (WsHeader *)a.ws, a.sorted, a8, asc, h8, hsc,
        yout, K, N, a.d.top_k, a.P, col_tiles, row_tiles, shared, shared ? a.T : 0,
        (size_t)(shared ? 1 : a.d.n_experts) * N * (size_t)(K / 2));
}

}  // namespace

hipError_t launch_prepare_mx8(const FwdArgs &a, hipStream_t s) {
    const Mx8Areas m = mx8_areas(a);
    constexpr int rows_per_block = kPrepThreads / kWave;   // one wavefront per token row
    prepare_mx8_kernel<<<1 + (a.T + rows_per_block - 1) / rows_per_block, kPrepThreads, 0, s>>>(
        a.offsets, a.d.n_experts, a.P, a.x, a.d.act_dtype == FW_BF16, a.d.hidden, a.T,
        a.L.max_tiles, (int4 *)(a.ws + a.L.active), (int4 *)(a.ws + a.L.tiles), m.x8, m.xs,
        (int *)(a.ws + a.L.split_cnt), (WsHeader *)a.ws);
    return hipGetLastError();
}

hipError_t launch_gemm_mx_gate_up(const FwdArgs &a, hipEvent_t routed_done, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const Mx8Areas m = mx8_areas(a);
    const size_t hr = (size_t)a.P * d.ffn;   // the shared expert's h rows start here
    launch_mx<true>(a, a.wg, a.wu, m.x8, m.xs, m.h8, m.hs, nullptr, d.hidden, d.ffn, 0, s);
    if (routed_done) (void)hipEventRecord(routed_done, s);
    if (d.shared_ffn > 0)
        launch_mx<true>(a, a.sg, a.su, m.x8, m.xs, m.h8 + hr, m.hs + hr / 32, nullptr, d.hidden,
                        d.shared_ffn, 1, s);
    return hipGetLastError();
}

hipError_t launch_gemm_mx_down(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const Mx8Areas m = mx8_areas(a);
    const size_t hr = (size_t)a.P * d.ffn;
    float *y = (float *)(a.ws + a.L.y);
    launch_mx<false>(a, a.wd, nullptr, m.h8, m.hs, nullptr, nullptr, y, d.ffn, d.hidden, 0, s);
    if (d.shared_ffn > 0)
        launch_mx<false>(a, a.sd, nullptr, m.h8 + hr, m.hs + hr / 32, nullptr, nullptr,
                         y + (size_t)a.P * d.hidden, d.shared_ffn, d.hidden, 1, s);
    return hipGetLastError();
}

}  // namespace fw
