// Forward, GEMM family (prefill-sized batches): grouped, dequant-fused expert
// GEMMs on MFMA.  Batched expert work is a dense contraction (the pages' runtime
// runs prefill experts through "the dense batch kernels" and block-table MMQ
// GEMMs -- Flyweight 0.2.0 "Features" and "Runtime controls"), so it runs on
// the matrix cores:
//
//  - a tile is up to 128 rows of one expert's segment of the sorted pair list
//    (tokens gathered through sorted_pairs) times 128 weight rows; the tile list
//    is built on the device (prepare kernel), so no host synchronisation;
//  - K advances 64 elements (two GGUF blocks) per step: the activation rows
//    (fp16) and the weight rows dequantised to fp16 (exact codes times the fp16
//    scale, one rounding) are staged in double-buffered, padded LDS, both in
//    the pair order of decode_pairs (the MFMA sums over K in any order, so
//    permuting K the same way on both operands changes nothing), which lets a
//    block dequantise with packed fp16 operations;
//  - v_mfma_f32_16x16x32_f16 with fp32 accumulation; four wavefronts in 2x2,
//    each owning 64 x 64 of the tile (4 x 4 MFMA tiles);
//  - gate/up: the 128 weight rows are 64 gate rows and the same 64 up rows,
//    arranged so a lane holds gate and up of the same (token, feature) and
//    forms SiLU(g)*u in registers; outputs leave through LDS as whole rows;
//  - the XCDs take the row tiles round-robin and consecutive workgroups of one
//    XCD take the column tiles of one row tile, so its gathered activation rows
//    stay in that XCD's L2;
//  - a wavefront whose 64 tile rows hold fewer valid rows runs a specialisation
//    with fewer MFMA row tiles (partial tiles of small experts cost less).
//
// fp16 rather than bf16 operands: bf16 (8-bit significand) roundings of the
// dequantised weights cost ~3e-3 relative error on a layer output, above the
// layer's tolerance; fp16 costs ~2.4e-4 at the same MFMA rate on gfx950.
#include <math.h>

#include "common.h"

namespace fw {
namespace {

constexpr int BM = kGemmBM;   // 128 token rows
constexpr int BN = 128;       // weight rows
constexpr int BK = 64;        // K per step (two blocks)
constexpr int LDK = BK + 8;   // padded LDS row (halfs): 144-byte stride
constexpr int kThreads = 256;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

struct Smem {
    _Float16 a[2][BM * LDK];
    _Float16 b[2][BN * LDK];
};
// the epilogues reuse the staging buffers: [BM][72] fp16 or [64][BN + 4] fp32
static_assert(sizeof(Smem) >= BM * 72 * 2 && sizeof(Smem) >= 64 * (BN + 4) * 4, "epilogue fits");

// Raw bytes of block kb of a weight row: the block pair starting at block
// 2*(kb/2) is 4-byte aligned; block kb occupies dwords [R*s, R*s + R) of the
// pair's window with R = 5 (Q4_0) or 9 (Q8_0), s = kb & 1.
template <int Q> struct Raw {
    uint32_t w[Q == FW_Q4_0 ? 5 : 9];
};

template <int Q>
__device__ __forceinline__ void fetch_block(const uint8_t *row, int kb, Raw<Q> &r) {
    constexpr int R = Q == FW_Q4_0 ? 5 : 9, PB = Q == FW_Q4_0 ? 36 : 68;
    const uint32_t *p = (const uint32_t *)(row + (size_t)(kb >> 1) * PB) + (R - 1) * (kb & 1);
#pragma unroll
    for (int i = 0; i < R; ++i) r.w[i] = p[i];
}

// The fetched block as 16 fp16 pairs in pair order (see decode_pairs), each
// pair value times the block scale: d * code rounded once to fp16 (pairs
// j = 1, 3 carry 16 * d * code, matched by activations stored / 16).
template <int Q>
__device__ __forceinline__ void dequant_block(const Raw<Q> &r, int s, uint32_t *dst) {
    constexpr int NQ = Q == FW_Q4_0 ? 4 : 8;
    uint32_t q[NQ];
    uint32_t dbits;
    if (s == 0) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) q[i] = funnel16(r.w[i], r.w[i + 1]);
        dbits = r.w[0] & 0xFFFFu;
    } else {
#pragma unroll
        for (int i = 0; i < NQ; ++i) q[i] = r.w[i + 1];
        dbits = r.w[0] >> 16;
    }
    h2 p[16];
    codes_to_pairs<Q>(q, p, pair_magic<Q>());
    const h2 d2 = as_h2(dbits | (dbits << 16));
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i] = __builtin_bit_cast(uint32_t, p[i] * d2);
}

// What one thread of a tile needs through the K loop and the epilogue.
struct TileCtx {
    const _Float16 *asrc[4];   // this thread's four activation rows, at its 16-byte chunk
    const uint8_t *bsrc;    // this thread's weight row
    _Float16 *hout;
    float *yout;
    int achunk, brow, bblk, wm, wn, lane, tid, steps, rows, rb, ct, N;
};

// The K loop and epilogue of one tile for a wavefront whose 64 tile rows hold
// MI 16-row MFMA tiles of valid rows (rows past the expert's segment cost no
// matrix work).  Every instantiation passes the same barriers in the same
// order, so waves of one workgroup may run different MI.
template <int Q, bool GU, int MI>
__device__ __forceinline__ void tile_run(Smem &sm, const TileCtx &c) {
    const _Float16 *const as0 = c.asrc[0], *const as1 = c.asrc[1], *const as2 = c.asrc[2],
                          *const as3 = c.asrc[3];
    const uint8_t *const bsrc = c.bsrc;
    const int achunk = c.achunk, brow = c.brow, bblk = c.bblk;
    const int wm = c.wm, wn = c.wn, lane = c.lane, tid = c.tid, steps = c.steps;
    const int rows = c.rows, rb = c.rb, ct = c.ct, N = c.N;

    // staging: the weight blocks of step s (from HBM) are fetched into
    // registers B[s % 4] during the MFMAs of step s-3, the activation rows
    // (mostly L2 hits) into A[s % 2] during step s-2; both are committed
    // (dequantised, registers -> LDS) after the MFMAs of step s-1
    u4 ra0[4], ra1[4];
    Raw<Q> rw0, rw1, rw2, rw3;
#define FW_FETCH_A(step, R)                                               \
    do {                                                                  \
        ra##R[0] = *(const u4 *)(as0 + (step) * BK);                      \
        ra##R[1] = *(const u4 *)(as1 + (step) * BK);                      \
        ra##R[2] = *(const u4 *)(as2 + (step) * BK);                      \
        ra##R[3] = *(const u4 *)(as3 + (step) * BK);                      \
    } while (0)
#define FW_FETCH_B(step, R) fetch_block<Q>(bsrc, 2 * (step) + bblk, rw##R)
#define FW_COMMIT(buf, RA, RB)                                                           \
    do {                                                                                 \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                                    \
            *(u4 *)&sm.a[buf][(tid / 8 + 32 * i) * LDK + achunk * 8] = ra##RA[i];            \
        uint32_t t[16];                                                                  \
        dequant_block<Q>(rw##RB, bblk, t);                                               \
        uint4 *bd = (uint4 *)&sm.b[buf][brow * LDK + bblk * 32];                         \
        bd[0] = uint4{t[0], t[1], t[2], t[3]};                                           \
        bd[1] = uint4{t[4], t[5], t[6], t[7]};                                           \
        bd[2] = uint4{t[8], t[9], t[10], t[11]};                                         \
        bd[3] = uint4{t[12], t[13], t[14], t[15]};                                       \
    } while (0)

    f4 acc[MI > 0 ? MI : 1][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    FW_FETCH_A(0, 0);
    FW_FETCH_A(1, 1);
    FW_FETCH_B(0, 0);
    FW_FETCH_B(1, 1);
    FW_FETCH_B(2, 2);
    FW_COMMIT(0, 0, 0);
    __syncthreads();
    const int fr = lane & 15, fk = (lane >> 4) * 8;   // fragment row / k offset
    for (int st = 0; st < steps; st += 4) {
        // step S: LDS buffer S % 2 holds S; fetch A(S+2) into A[S % 2] and
        // B(S+3) into B[(S+3) % 4] (clamped: no conditional writes); commit S+1
#define FW_STEP(S, BUF, RA_F, RB_F, RA_N, RB_N)                                                 \
        {                                                                                       \
            FW_FETCH_A(min((S) + 2, steps - 1), RA_F);                                          \
            FW_FETCH_B(min((S) + 3, steps - 1), RB_F);                                          \
            if constexpr (MI > 0) {                                                             \
                _Pragma("unroll") for (int kk = 0; kk < BK; kk += 32) {                         \
                    h8 af[MI > 0 ? MI : 1], bf[4];                                              \
                    _Pragma("unroll") for (int j = 0; j < 4; ++j)                               \
                        bf[j] = *(const h8 *)&sm.b[BUF][(wn * 64 + j * 16 + fr) * LDK + kk + fk]; \
                    _Pragma("unroll") for (int i = 0; i < MI; ++i)                              \
                        af[i] = *(const h8 *)&sm.a[BUF][(wm * 64 + i * 16 + fr) * LDK + kk + fk]; \
                    _Pragma("unroll") for (int i = 0; i < MI; ++i)                              \
                        _Pragma("unroll") for (int j = 0; j < 4; ++j)                           \
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j],    \
                                                                               acc[i][j], 0, 0, 0); \
                }                                                                               \
            }                                                                                   \
            if ((S) + 1 < steps) FW_COMMIT((BUF) ^ 1, RA_N, RB_N);                              \
            __syncthreads();                                                                    \
        }
        FW_STEP(st, 0, 0, 3, 1, 1)
        FW_STEP(st + 1, 1, 1, 0, 0, 2)
        FW_STEP(st + 2, 0, 0, 1, 1, 3)
        FW_STEP(st + 3, 1, 1, 2, 0, 0)
#undef FW_STEP
    }

#undef FW_FETCH_A
#undef FW_FETCH_B
#undef FW_COMMIT

    // ---- epilogue through LDS (the staging buffers are free now) ----
    // acc[i][j][r]: tile row wm*64 + i*16 + 4*(lane/16) + r, column wn*64 + j*16 + lane%16
    if constexpr (GU) {
        // a(row, feature) with feature index wn*32 + j*16 + lane%16, j = 0,1
        // [BM][OH] fp16; the 8-half pad keeps rows 4 apart off the same banks
        constexpr int OH = 72;
        _Float16 *o = (_Float16 *)&sm;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float g = acc[i][j][r], u = acc[i][j + 2][r];   // gate, up
                    const int row = wm * 64 + i * 16 + 4 * (lane >> 4) + r;
                    const int col = wn * 32 + j * 16 + (lane & 15);
                    float a = g / (1.0f + __expf(-g)) * u;
                    if (col & 16) a *= 0.0625f;   // pair order: pairs j = 1, 3 hold value / 16
                    o[row * OH + (col & ~31) + pair_pos(col & 31)] = (_Float16)a;
                }
        __syncthreads();
        // 128 rows x 128 bytes: thread -> (row tid/2, 64 bytes)
        const int row = tid >> 1, part = tid & 1;
        if (row < rows) {
            const uint4 *s = (const uint4 *)&o[row * OH + part * 32];
            uint4 *d = (uint4 *)(c.hout + (size_t)(rb + row) * N + ct * 64 + part * 32);
#pragma unroll
            for (int i = 0; i < 4; ++i) d[i] = s[i];
        }
    } else {
        // fp32 outputs in two passes of 64 rows
        // [64][OF] fp32; the 4-float pad keeps rows 4 apart off the same banks
        constexpr int OF = BN + 4;
        float *o = (float *)&sm;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (wm == half) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int row = i * 16 + 4 * (lane >> 4) + r;
                            const int col = wn * 64 + j * 16 + (lane & 15);
                            o[row * OF + col] = acc[i][j][r];
                        }
            }
            __syncthreads();
            // 64 rows x 512 bytes: thread -> (row tid/4, 128 bytes)
            const int row = tid >> 2, part = tid & 3;
            const int grow = half * 64 + row;
            if (grow < rows) {
                const uint4 *s = (const uint4 *)&o[row * OF + part * 32];
                uint4 *d = (uint4 *)(c.yout + (size_t)(rb + grow) * N + ct * BN + part * 32);
#pragma unroll
                for (int i = 0; i < 8; ++i) d[i] = s[i];
            }
            __syncthreads();
        }
    }
}

// One (row tile, column tile) of one expert (or of the shared expert).
//  GU:  A = x rows gathered through sorted_pairs (routed) or token rows
//       (shared); weight rows = 64 gate + 64 up features; writes
//       a = SiLU(g) * u (fp16, pair order) for 64 features;
//  !GU: A = rows of a (fp16); weight rows = 128 outputs; writes y (fp32).
template <int Q, bool GU>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint8_t *__restrict__ wa, const uint8_t *__restrict__ wb,
    const int4 *__restrict__ tiles, WsHeader *__restrict__ hdr,
    const int32_t *__restrict__ sorted, const _Float16 *__restrict__ ain,
    _Float16 *__restrict__ hout, float *__restrict__ yout, int K, int N, int k, int P,
    int col_tiles, int n_row_tiles_max, int shared, int shared_rows) {
    __shared__ Smem sm;
    // XCD-aware order: workgroup b runs on XCD b % 8; the XCDs take the row
    // tiles round-robin (so the device-built list, a prefix of the row tiles,
    // spreads over all eight), and consecutive workgroups of one XCD take the
    // column tiles of one row tile (its gathered activation rows stay in that
    // XCD's L2).
    const int xcd = blockIdx.x % 8, i = blockIdx.x / 8;
    const int rt = (i / col_tiles) * 8 + xcd, ct = i % col_tiles;
    if (rt >= n_row_tiles_max) return;
    int expert = 0, rb = 0, rows = 0;
    if (shared) {
        rb = rt * BM;
        rows = min(BM, shared_rows - rb);
        if (rows <= 0) return;
    } else {
        if (rt >= ld_const(&hdr->n_tiles)) return;
        const int4 tl = ld_const(tiles + rt);   // (expert, first row, rows)
        expert = tl.x;
        rb = tl.y;
        rows = tl.z;
    }
    const size_t rowbytes = (size_t)(K / 32) * QT<Q>::kBlockBytes;
    const size_t esz = (size_t)N * rowbytes;
    TileCtx c;
    c.tid = threadIdx.x;
    c.lane = c.tid % kWave;
    const int wave = wave_id();
    c.wm = wave >> 1;
    c.wn = wave & 1;

    // ---- per-thread load roles (fixed over the K loop) ----
    // A: thread -> 16-byte chunk tid % 8 of tile rows tid/8 + 32 i, i < 4 (eight
    // lanes read a row's 128 bytes of a K step together)
    c.achunk = c.tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int arow = c.tid / 8 + 32 * i;
        const int r = rb + min(arow, rows - 1);
        int src_row = r;
        if (GU && !shared) {
            const int q = ld_const(sorted + r);
            if ((unsigned)q >= (unsigned)P) {
                if (arow < rows) atomicOr(&hdr->status, FW_STATUS_BAD_PAIR);
                src_row = 0;
            } else {
                src_row = q / k;
            }
        }
        c.asrc[i] = ain + (size_t)src_row * K + c.achunk * 8;
    }
    // B: thread -> weight row tid/2 of the tile, block (tid&1) of the step
    c.brow = c.tid >> 1;
    c.bblk = c.tid & 1;
    if (GU) {
        // tile rows: wn*64 + [0,32) gate features, wn*64 + [32,64) up features,
        // features ct*64 + wn*32 + [0,32)
        const int grp = c.brow >> 6, within = c.brow & 63;
        const int f = ct * 64 + grp * 32 + (within & 31);
        const uint8_t *base = (within < 32) ? wa : wb;
        c.bsrc = base + (size_t)expert * esz + (size_t)f * rowbytes;
    } else {
        c.bsrc = wa + (size_t)expert * esz + (size_t)(ct * BN + c.brow) * rowbytes;
    }
    c.hout = hout;
    c.yout = yout;
    c.steps = K / BK;   // a multiple of 4 (K is a multiple of 256)
    c.rows = rows;
    c.rb = rb;
    c.ct = ct;
    c.N = N;
    // 16-row MFMA tiles of this wave that hold valid rows
    const int mi = (min(max(rows - c.wm * 64, 0), 64) + 15) / 16;
    switch (mi) {
        case 4: tile_run<Q, GU, 4>(sm, c); break;
        case 3: tile_run<Q, GU, 3>(sm, c); break;
        case 2: tile_run<Q, GU, 2>(sm, c); break;
        case 1: tile_run<Q, GU, 1>(sm, c); break;
        default: tile_run<Q, GU, 0>(sm, c); break;
    }
}

template <int Q, bool GU>
void launch(const FwdArgs &a, const uint8_t *wa, const uint8_t *wb, const _Float16 *ain,
            _Float16 *hout, float *yout, int K, int N, int shared, hipStream_t s) {
    const int col_tiles = GU ? N / 64 : N / BN;
    // routed: at most one partial tile per expert (the device list may hold
    // fewer; the surplus workgroups return at once)
    const int row_tiles = shared ? (a.T + BM - 1) / BM
                                 : std::min(a.L.max_tiles, (a.P + BM - 1) / BM + a.d.n_experts);
    const int nblk = (row_tiles + 7) / 8 * 8 * col_tiles;   // eight XCDs x whole row tiles
    gemm_kernel<Q, GU><<<nblk, kThreads, 0, s>>>(
        wa, wb, (const int4 *)(a.ws + a.L.tiles), (WsHeader *)a.ws, a.sorted, ain, hout, yout,
        K, N, a.d.top_k, a.P, col_tiles, row_tiles, shared, shared ? a.T : 0);
}

}  // namespace

hipError_t launch_gemm_gate_up(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const _Float16 *x = (const _Float16 *)(a.ws + a.L.x16);
    _Float16 *h = (_Float16 *)(a.ws + a.L.h);
    if (d.expert_q == FW_Q4_0)
        launch<FW_Q4_0, true>(a, a.wg, a.wu, x, h, nullptr, d.hidden, d.ffn, 0, s);
    else
        launch<FW_Q8_0, true>(a, a.wg, a.wu, x, h, nullptr, d.hidden, d.ffn, 0, s);
    if (d.shared_ffn > 0) {
        _Float16 *hsh = h + (size_t)a.P * d.ffn;
        if (d.shared_q == FW_Q4_0)
            launch<FW_Q4_0, true>(a, a.sg, a.su, x, hsh, nullptr, d.hidden, d.shared_ffn, 1, s);
        else
            launch<FW_Q8_0, true>(a, a.sg, a.su, x, hsh, nullptr, d.hidden, d.shared_ffn, 1, s);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_down(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const _Float16 *h = (const _Float16 *)(a.ws + a.L.h);
    float *y = (float *)(a.ws + a.L.y);
    if (d.expert_q == FW_Q4_0)
        launch<FW_Q4_0, false>(a, a.wd, nullptr, h, nullptr, y, d.ffn, d.hidden, 0, s);
    else
        launch<FW_Q8_0, false>(a, a.wd, nullptr, h, nullptr, y, d.ffn, d.hidden, 0, s);
    if (d.shared_ffn > 0) {
        const _Float16 *hsh = h + (size_t)a.P * d.ffn;
        float *ysh = y + (size_t)a.P * d.hidden;
        if (d.shared_q == FW_Q4_0)
            launch<FW_Q4_0, false>(a, a.sd, nullptr, hsh, nullptr, ysh, d.shared_ffn, d.hidden, 1, s);
        else
            launch<FW_Q8_0, false>(a, a.sd, nullptr, hsh, nullptr, ysh, d.shared_ffn, d.hidden, 1, s);
    }
    return hipGetLastError();
}

}  // namespace fw
