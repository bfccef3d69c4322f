// Forward, GEMM family (prefill-sized batches), register-dequant form: grouped
// expert GEMMs on MFMA whose weights never pass through LDS.
//
//  - a workgroup tile is up to 64 rows of one expert's segment of the sorted
//    pair list (tokens gathered through sorted_pairs) times 256 weight rows;
//    each of the four wavefronts owns 64 weight rows (four 16-row MFMA column
//    groups) and all 64 token rows (four 16-row MFMA row groups; a tile with
//    fewer rows runs only the row groups that hold rows: 1, 2 or 4);
//  - K advances one 256-element unit (8 GGUF blocks) per step.  In the MFMA's
//    k order, lane group g = lane / 16 covers blocks 2g and 2g + 1 of the unit
//    and slice i (0..7) of a step covers block 2g + i / 4, fp16 pairs
//    4 (i % 4) .. 4 (i % 4) + 3 in the pair order of decode_pairs (the MFMA
//    sums over k in any order, so the activations are laid out the same way);
//  - weights: lane (n = lane % 16, g) loads the 36-byte (Q4_0) or 68-byte
//    (Q8_0) window of blocks 2g, 2g + 1 of its weight row (dword aligned) and
//    turns one code dword into the four fp16 pairs of a B fragment (exact code
//    times the fp16 scale, one rounding) right before the MFMAs that use it;
//    no LDS traffic, no bank conflicts.  Q4_0 windows are loaded one step
//    ahead into a second buffer; the wider Q8_0 and Q4_K windows (17 and 12
//    dwords per column group) have one buffer, refilled after the step's
//    MFMAs, which keeps those kernels within 256 VGPRs at two waves per SIMD
//    (with two buffers they spilled into AGPRs at one wave per SIMD: Q4_K
//    prefill T=2048 545 -> 446 us, Q8_0 560 -> 515 us);
//  - activations: the 64 x 256 fp16 tile of a step is staged through
//    double-buffered, padded LDS (32 lanes read one row's 512 bytes together),
//    loaded one step ahead; A fragments are read per slice;
//  - v_mfma_f32_16x16x32_f16 with fp32 accumulation; gate/up: a wavefront's 64
//    weight rows are 32 gate and the same 32 up features, so a lane holds gate
//    and up of the same (token, feature) and forms SiLU(g)*u in registers;
//    that fp16 output (in pair order) leaves through LDS as whole rows, while
//    the down projection's fp32 rows go straight from the accumulators to
//    memory, 64 contiguous bytes per 16 lanes (through LDS they took a
//    barrier and a 66 KB round trip per tile: prefill T=2048 down 117 -> 103
//    us);
//  - each XCD takes a contiguous eighth of the row-tile list, so the row tiles
//    of one expert share an L2 and its weights are fetched about once;
//    consecutive workgroups of one XCD take the column tiles of one row tile.
#include <math.h>

#include "common.h"

namespace fw {
namespace {

constexpr int BM = kGemm2BM;   // token rows per tile (a multiple of 64)
constexpr int kMaxMI = BM / 16;   // 16-row MFMA row groups per tile
constexpr int BN = 256;        // weight rows per workgroup
constexpr int BK = kUnit;      // 256 elements per step
constexpr int LDA = BK + 8;    // padded LDS activation row (halfs): 528 bytes
constexpr int kThreads = 256;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

struct Smem2 {
    _Float16 a[2][BM * LDA];
};
// epilogues reuse the activation buffers: [BM][136] fp16 or [BM][260] fp32
static_assert(sizeof(Smem2) >= BM * 136 * 2 && sizeof(Smem2) >= BM * (BN + 4) * 4,
              "epilogue fits");

// Dwords of the window of blocks 2g, 2g + 1 of a unit, per weight row.
// Q4_K: the super-block's 16-byte header and the 32 code bytes of group g.
template <int Q> constexpr int win_dwords() { return Q == FW_Q4_0 ? 9 : Q == FW_Q4_K ? 12 : 17; }

// p: the lane's window (Q8_0 / Q4_0) or its row's unit (Q4_K, whose code bytes
// sit qoff bytes in).
template <int Q>
__device__ __forceinline__ void load_window(const uint8_t *p, uint32_t qoff, uint32_t *w) {
    const uint32_t *q = (const uint32_t *)p;
    if constexpr (Q == FW_Q4_K) {
        const uint32_t *c = (const uint32_t *)(p + qoff);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = q[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[4 + i] = c[i];
    } else {
#pragma unroll
        for (int i = 0; i < win_dwords<Q>(); ++i) w[i] = q[i];
    }
}

// Per-step constants of a Q4_K window (sub-blocks A = 2g, B = 2g + 1 of the
// lane's group g), as fp32 bits: k[2h] = d * scale, k[2h + 1] = -dmin * min
// (both exact in fp32).
__device__ __forceinline__ void q4k_consts(const uint32_t *w, int g, uint32_t *k) {
    const float d = half_bits_to_float(w[0] & 0xFFFFu), dmin = half_bits_to_float(w[0] >> 16);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int j = 2 * g + h, jj = (j - 4) & 3;
        const uint32_t lo_s = __builtin_amdgcn_ubfe(w[1], 8 * j, 6);
        const uint32_t lo_m = __builtin_amdgcn_ubfe(w[2], 8 * j, 6);
        const uint32_t hi_s = __builtin_amdgcn_ubfe(w[3], 8 * jj, 4) |
                              __builtin_amdgcn_ubfe(w[1], 8 * jj + 6, 2) << 4;
        const uint32_t hi_m = __builtin_amdgcn_ubfe(w[3], 8 * jj + 4, 4) |
                              __builtin_amdgcn_ubfe(w[2], 8 * jj + 6, 2) << 4;
        const uint32_t sc = j < 4 ? lo_s : hi_s, mn = j < 4 ? lo_m : hi_m;
        k[2 * h] = __float_as_uint(d * (float)sc);
        k[2 * h + 1] = __float_as_uint(-dmin * (float)mn);
    }
}

// Largest block-scale magnitude (fp16 bits) of a Q4_0 / Q8_0 window's two blocks.
template <int Q>
__device__ __forceinline__ uint32_t d_bits(const uint32_t *w) {
    constexpr int hi = Q == FW_Q4_0 ? 4 : 8;   // dword holding the odd block's scale
    return max(w[0] & 0x7FFFu, __builtin_amdgcn_ubfe(w[hi], 16, 15));
}

// Bound on the 16x-scaled magnitude of a Q4_K window's weights from its
// per-step constants: 16 (15 |d scale| + |dmin min|) over both sub-blocks.
__device__ __forceinline__ float q4k_bound(const uint32_t *k) {
    float b = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
        b = fmaxf(b, 16.0f * fmaf(15.0f, fabsf(__uint_as_float(k[2 * h])),
                                  fabsf(__uint_as_float(k[2 * h + 1]))));
    return b;
}

// B fragment of slice I from a Q4_K window: sub-block H = I / 4 of the group,
// pairs 4 (I % 4) .. + 3.  Each weight d * scale * q - dmin * min is formed in
// fp32 (exact up to one fp32 rounding) and rounded once to fp16, like a Q4_0
// weight; pairs j = 1, 3 then carry 16x (exact).
template <int I>
__device__ __forceinline__ h8 frag_b_q4k(const uint32_t *w, const uint32_t *k) {
    constexpr int H = I / 4, m = I % 4;
    const uint32_t c0 = w[4 + m] >> (4 * H), c1 = w[8 + m] >> (4 * H);
    const uint32_t a0 = c0 & 0x0F0F0F0Fu, a1 = c1 & 0x0F0F0F0Fu;   // elements 4m.., 16+4m..
    const float ds = __uint_as_float(k[2 * H]), nd = __uint_as_float(k[2 * H + 1]);
    // (float)((v >> 8b) & 255) is one v_cvt_f32_ubyte<b>
    auto e = [&](uint32_t v, int byte) {
        return (_Float16)fmaf((float)((v >> (8 * byte)) & 255u), ds, nd);
    };
    const h2 k16 = {(_Float16)16.0f, (_Float16)16.0f};
    h2 p[4];
    p[0] = h2{e(a0, 0), e(a0, 2)};
    p[1] = h2{e(a1, 0), e(a1, 2)} * k16;
    p[2] = h2{e(a0, 1), e(a0, 3)};
    p[3] = h2{e(a1, 1), e(a1, 3)} * k16;
    h8 f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = p[j][0];
        f[2 * j + 1] = p[j][1];
    }
    return f;
}

// B fragment of slice I from a window: block I / 4 of the pair (even: 2 bytes
// into the window, odd: dword aligned), pairs 4 (I % 4) .. + 3, times the
// block's fp16 scale.
template <int Q, int I>
__device__ __forceinline__ h8 frag_b(const uint32_t *w) {
    constexpr int m = I % 4;
    uint32_t dbits, c0, c1 = 0;
    if constexpr (Q == FW_Q4_0) {
        if constexpr (I < 4) {
            dbits = w[0] & 0xFFFFu;
            c0 = funnel16(w[m], w[m + 1]);
        } else {
            dbits = w[4] >> 16;
            c0 = w[5 + m];
        }
    } else {
        if constexpr (I < 4) {
            dbits = w[0] & 0xFFFFu;
            c0 = funnel16(w[m], w[m + 1]);
            c1 = funnel16(w[4 + m], w[5 + m]);
        } else {
            dbits = w[8] >> 16;
            c0 = w[9 + m];
            c1 = w[13 + m];
        }
    }
    const uint32_t magic = pair_magic<Q>();
    h2 p[4];
    if constexpr (Q == FW_Q4_0) {
        const h2 k1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
        const h2 k1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
        const uint32_t c8 = c0 >> 8;
        p[0] = as_h2(and_or(c0, 0x000F000Fu, magic)) - k1032;
        p[1] = as_h2(and_or(c0, 0x00F000F0u, magic)) - k1152;
        p[2] = as_h2(and_or(c8, 0x000F000Fu, magic)) - k1032;
        p[3] = as_h2(and_or(c8, 0x00F000F0u, magic)) - k1152;
    } else {
        const h2 k1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
        const h2 k16 = {(_Float16)16.0f, (_Float16)16.0f};
        const h2 k18432 = {(_Float16)18432.0f, (_Float16)18432.0f};
        const uint32_t lo = c0 ^ 0x80808080u, hi = c1 ^ 0x80808080u;
        p[0] = as_h2(__builtin_amdgcn_perm(magic, lo, 0x04020400u)) - k1152;
        p[1] = as_h2(__builtin_amdgcn_perm(magic, hi, 0x04020400u)) * k16 - k18432;
        p[2] = as_h2(__builtin_amdgcn_perm(magic, lo, 0x04030401u)) - k1152;
        p[3] = as_h2(__builtin_amdgcn_perm(magic, hi, 0x04030401u)) * k16 - k18432;
    }
    const h2 d2 = as_h2(dbits | (dbits << 16));
    h8 f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const h2 v = p[j] * d2;
        f[2 * j] = v[0];
        f[2 * j + 1] = v[1];
    }
    return f;
}

// B fragment of slice I of any format (kq: the Q4_K per-step constants).
template <int Q, int I>
__device__ __forceinline__ h8 frag_any(const uint32_t *w, const uint32_t *kq) {
    if constexpr (Q == FW_Q4_K)
        return frag_b_q4k<I>(w, kq);
    else
        return frag_b<Q, I>(w);
}

struct Tile2 {
    const _Float16 *abase;     // activation rows (uniform)
    uint32_t aoff[BM / 8];     // this thread's rows, at its 16-byte chunk: element offsets
    const uint8_t *bbase[2];   // the expert's weight matrices (uniform): gate/up or down
    uint32_t boff[4];          // this lane's rows (col groups), at its block pair: byte offsets
    uint32_t qoff;             // Q4_K: byte offset of the lane's code group in a unit
    _Float16 *hout;
    float *yout;
    // row exponents: gate/up reads the token's x exponent (iexp[token]; the
    // token of a routed row via sorted) and records 2x it per h row in oexp;
    // the down projection reads iexp[row]
    const int32_t *sorted, *iexp;
    int32_t *oexp;
    WsHeader *hdr;
    int tid, lane, wave, steps, rows, rb, ct, N, k, P, shared;
};

// The K loop and epilogue of one tile, MI 16-row groups of token rows.  The
// kernel's register count is that of the largest MI; the smaller ones skip
// the MFMAs and activation loads of a partial tile's empty row groups.
template <int Q, bool GU, int MI>
__device__ __forceinline__ void tile2_run(Smem2 &sm, const Tile2 &c) {
    constexpr int WD = win_dwords<Q>();
    constexpr int UB = QT<Q>::kUnitBytes;
    const int lane = c.lane, tid = c.tid, steps = c.steps;
    const int g = lane >> 4, fr = lane & 15;

    f4 acc[MI > 0 ? MI : 1][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    constexpr int NA = 2 * MI;   // activation chunks per thread: rows tid / 32 + 8 j
    u4 ra[NA];                   // activation chunks of the next step
    uint32_t wb0[4][WD], wb1[4][WD];   // weight windows: this step / next step
    uint32_t dmax = 0;           // largest block-scale magnitude bits met (Q8_0 / Q4_0)
    float wmax = 0.f;            // largest Q4_K weight bound met

    auto load_a = [&](int st) {
#pragma unroll
        for (int j = 0; j < NA; ++j) ra[j] = *(const u4 *)(c.abase + c.aoff[j] + st * BK);
    };
    auto commit_a = [&](int buf) {
#pragma unroll
        for (int j = 0; j < NA; ++j)
            *(u4 *)&sm.a[buf][(tid / 32 + 8 * j) * LDA + (tid & 31) * 8] = ra[j];
    };
#define FW_LOAD_B(W, st)                                                   \
    _Pragma("unroll") for (int cg = 0; cg < 4; ++cg)                       \
        load_window<Q>(c.bbase[GU ? cg >> 1 : 0] + c.boff[cg] + (st) * UB, c.qoff, W[cg]);

    // one step: 8 slices x 4 column groups x MI row groups of MFMAs; the A
    // fragments of slice i + 1 are read from LDS while slice i's MFMAs run
#define FW_FRAG_B(I, CG, W)                                                                  \
    (I == 0 ? frag_any<Q, 0>(W[CG], kq[CG]) : I == 1 ? frag_any<Q, 1>(W[CG], kq[CG])          \
     : I == 2 ? frag_any<Q, 2>(W[CG], kq[CG]) : I == 3 ? frag_any<Q, 3>(W[CG], kq[CG])        \
     : I == 4 ? frag_any<Q, 4>(W[CG], kq[CG]) : I == 5 ? frag_any<Q, 5>(W[CG], kq[CG])        \
     : I == 6 ? frag_any<Q, 6>(W[CG], kq[CG]) : frag_any<Q, 7>(W[CG], kq[CG]))
#define FW_MMA(BUF, W)                                                                        \
    if constexpr (MI > 0) {                                                                   \
        uint32_t kq[4][4];                                                                    \
        if constexpr (Q == FW_Q4_K)                                                           \
            _Pragma("unroll") for (int cg = 0; cg < 4; ++cg) {                                \
                q4k_consts(W[cg], g, kq[cg]);                                                 \
                wmax = fmaxf(wmax, q4k_bound(kq[cg]));                                        \
            }                                                                                 \
        else                                                                                  \
            _Pragma("unroll") for (int cg = 0; cg < 4; ++cg) dmax = max(dmax, d_bits<Q>(W[cg])); \
        const _Float16 *abase = &sm.a[BUF][fr * LDA + 64 * g];                                \
        h8 afc[MI > 0 ? MI : 1], afn[MI > 0 ? MI : 1];                                        \
        _Pragma("unroll") for (int r = 0; r < MI; ++r)                                        \
            afc[r] = *(const h8 *)(abase + 16 * r * LDA);                                     \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                       \
            if (i < 7)                                                                        \
                _Pragma("unroll") for (int r = 0; r < MI; ++r)                                \
                    afn[r] = *(const h8 *)(abase + 16 * r * LDA + 8 * (i + 1));               \
            _Pragma("unroll") for (int cg = 0; cg < 4; ++cg) {                                \
                const h8 bf = FW_FRAG_B(i, cg, W);                                            \
                _Pragma("unroll") for (int r = 0; r < MI; ++r)                                \
                    acc[r][cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afc[r], bf, acc[r][cg], \
                                                                        0, 0, 0);             \
            }                                                                                 \
            _Pragma("unroll") for (int r = 0; r < MI; ++r) afc[r] = afn[r];                   \
            /* one slice's B fragments live at a time */                                     \
            __builtin_amdgcn_sched_barrier(0);                                                \
        }                                                                                     \
    }

    load_a(0);
    FW_LOAD_B(wb0, 0);
    commit_a(0);
    load_a(min(1, steps - 1));
    __syncthreads();
    // step s: LDS buffer s % 2 holds the activations of s, wb[s % 2] its
    // weights; the next step's weights are loaded first, the activations of
    // s + 1 committed and those of s + 2 loaded after the MFMAs (clamped loads
    // past the last step are redundant, never conditional)
    int st = 0;
    if constexpr (Q != FW_Q4_0) {
        // wide windows (Q8_0, Q4_K): one weight buffer, the next step's
        // windows loaded after this step's MFMAs; LDS buffer st % 2 holds
        // step st's activations, and buffer (st + 1) % 2 is refilled only
        // after the barrier that ends step st - 1's reads of it
        for (; st < steps; ++st) {
            const int cur = st & 1;
            FW_MMA(cur, wb0)
            FW_LOAD_B(wb0, min(st + 1, steps - 1));
            commit_a(cur ^ 1);
            load_a(min(st + 2, steps - 1));
            __syncthreads();
        }
    } else {
    for (; st + 1 < steps; st += 2) {
        FW_LOAD_B(wb1, st + 1);
        FW_MMA(0, wb0)
        commit_a(1);
        load_a(min(st + 2, steps - 1));
        __syncthreads();
        FW_LOAD_B(wb0, min(st + 2, steps - 1));
        FW_MMA(1, wb1)
        commit_a(0);
        load_a(min(st + 3, steps - 1));
        __syncthreads();
    }
    if (st < steps) {   // odd step count: the last step sits in buffer 0 / wb0
        FW_MMA(0, wb0)
        __syncthreads();
    }
    }
#undef FW_LOAD_B
#undef FW_MMA
#undef FW_FRAG_B

    // ---- epilogue through LDS (the activation buffers are free now) ----
    // acc[r][cg][j]: token row 16 r + 4 g + j, weight row 64 wave + 16 cg + fr
    const int rows = c.rows, rb = c.rb, ct = c.ct, N = c.N, wave = c.wave;
    // a dequantised weight beyond fp16 (16x-scaled extreme code): the outputs
    // of this tile are not reliable
    const bool wbad = Q == FW_Q4_K ? !(wmax <= 65504.0f)
                                   : dmax > (Q == FW_Q4_0 ? kQ4DMaxBits : kQ8DMaxBits);
    bool range = wbad;
    // each accumulator row's exponent (rows past the tile's end read its last row)
    int ex[MI > 0 ? MI : 1][4];
#pragma unroll
    for (int r = 0; r < MI; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = rb + min(16 * r + 4 * g + j, rows - 1);
            int src = rr;
            if (GU && !c.shared) {
                const int q = c.sorted[rr];
                src = (unsigned)q < (unsigned)c.P ? q / c.k : 0;
            }
            ex[r][j] = c.iexp[src];
        }
    if constexpr (GU) {
        // a(token, feature) for the workgroup's 128 features: [BM][OH] fp16;
        // g and u at the token's own scale (exact), SwiGLU in fp32, h stored at
        // 2^(2e) (pairs j = 1, 3 at 1/16)
        constexpr int OH = 136;
        _Float16 *o = (_Float16 *)&sm;
#pragma unroll
        for (int r = 0; r < MI; ++r)
#pragma unroll
            for (int cg = 0; cg < 2; ++cg)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = ex[r][j];
                    const float gv = __builtin_amdgcn_ldexpf(acc[r][cg][j], -e);
                    const float up = __builtin_amdgcn_ldexpf(acc[r][cg + 2][j], -e);
                    const int row = 16 * r + 4 * g + j;
                    const int col = 32 * wave + 16 * cg + fr;   // feature within the tile
                    const float a = gv / (1.0f + __expf(-gv)) * up;
                    const _Float16 ah =
                        (_Float16)__builtin_amdgcn_ldexpf(a, 2 * e - ((col & 16) ? 4 : 0));
                    range |= row < rows && (__builtin_bit_cast(uint16_t, ah) & 0x7C00u) == 0x7C00u;
                    o[row * OH + (col & ~31) + pair_pos(col & 31)] = ah;
                }
        // h rows' exponents, once per row
        if (ct == 0 && wave == 0 && fr == 0) {
#pragma unroll
            for (int r = 0; r < MI; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * r + 4 * g + j;
                    if (row < rows) c.oexp[rb + row] = 2 * ex[r][j];
                }
        }
        if (range) atomicOr(&c.hdr->status, FW_STATUS_RANGE);
        __syncthreads();
        // rows x 256 bytes: thread -> (row r0 + tid / 4, 64 bytes)
        const int part = tid & 3;
#pragma unroll
        for (int r0 = 0; r0 < 16 * MI; r0 += 64) {
            const int row = r0 + (tid >> 2);
            if (row < rows) {
                const uint4 *s = (const uint4 *)&o[row * OH + part * 32];
                uint4 *d = (uint4 *)(c.hout + (size_t)(rb + row) * N + ct * 128 + part * 32);
#pragma unroll
                for (int i = 0; i < 4; ++i) d[i] = s[i];
            }
        }
    } else {
        if (range) atomicOr(&c.hdr->status, FW_STATUS_RANGE);
        // y rows straight from the accumulators at the row's scale: for each
        // (row group, j, cg) the 16 lanes of a lane group write 64 contiguous
        // bytes of one row
#pragma unroll
        for (int r = 0; r < MI; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * r + 4 * g + j;
                if (row < rows) {
                    float *d = c.yout + (size_t)(rb + row) * N + ct * BN + 64 * wave + fr;
#pragma unroll
                    for (int cg = 0; cg < 4; ++cg)
                        d[16 * cg] = __builtin_amdgcn_ldexpf(acc[r][cg][j], -ex[r][j]);
                }
            }
    }
}

// One (row tile, column tile) of one expert (or of the shared expert).
//  GU:  A = x rows gathered through sorted_pairs (routed) or token rows
//       (shared); weight rows = 128 gate + 128 up features; writes
//       a = SiLU(g) * u (fp16, pair order) for 128 features;
//  !GU: A = rows of a (fp16); weight rows = 256 outputs; writes y (fp32).
template <int Q, bool GU>
__global__ __launch_bounds__(kThreads) void gemm2_kernel(
    const uint8_t *__restrict__ wa, const uint8_t *__restrict__ wb,
    const int4 *__restrict__ tiles, WsHeader *__restrict__ hdr,
    const int32_t *__restrict__ sorted, const _Float16 *__restrict__ ain,
    _Float16 *__restrict__ hout, float *__restrict__ yout, int K, int N, int k, int P,
    int col_tiles, int n_row_tiles_max, int shared, int shared_rows,
    const int32_t *__restrict__ iexp, int32_t *__restrict__ oexp) {
    __shared__ Smem2 sm;
    // XCD-aware order: workgroup b runs on XCD b % 8.  Each XCD takes a
    // contiguous eighth of the row tiles (the tiles of one expert are
    // consecutive, so they share that XCD's L2 and its weights are fetched
    // about once), column tiles fastest.
    const int xcd = blockIdx.x % 8, bi = blockIdx.x / 8;
    const int n_rt = shared ? (shared_rows + BM - 1) / BM
                            : min(ld_const(&hdr->n_tiles), n_row_tiles_max);
    const int per = (n_rt + 7) / 8;
    const int rl = bi / col_tiles, ct = bi % col_tiles;
    if (rl >= per) return;
    const int rt = xcd * per + rl;
    if (rt >= n_rt) return;
    int expert = 0, rb = 0, rows = 0;
    if (shared) {
        rb = rt * BM;
        rows = min(BM, shared_rows - rb);
    } else {
        const int4 tl = ld_const(tiles + rt);   // (expert, first row, rows)
        expert = tl.x;
        rb = tl.y;
        rows = tl.z;
    }
    const size_t rowbytes = (size_t)(K / 32) * QT<Q>::kBlockBytes;
    const size_t esz = (size_t)N * rowbytes;
    Tile2 c;
    c.tid = threadIdx.x;
    c.lane = c.tid % kWave;
    c.wave = wave_id();
    // activations: thread -> 16-byte chunk tid % 32 of tile rows tid / 32 + 8 j
#pragma unroll
    for (int j = 0; j < BM / 8; ++j) {
        const int arow = c.tid / 32 + 8 * j;
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
        c.aoff[j] = (uint32_t)src_row * K + (c.tid & 31) * 8;
    }
    // weights: lane -> row 16 cg + lane % 16 of the wave's 64, block pair lane / 16
    const int n = c.lane & 15, g = c.lane >> 4;
    c.abase = ain;
    c.bbase[0] = wa + (size_t)expert * esz;
    c.bbase[1] = GU ? wb + (size_t)expert * esz : c.bbase[0];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
        const int row = GU ? ct * 128 + 32 * c.wave + 16 * (cg & 1) + n   // feature (gate cg < 2)
                           : ct * BN + 64 * c.wave + 16 * cg + n;          // output row
        c.boff[cg] = (uint32_t)(row * rowbytes) + (Q == FW_Q4_K ? 0 : g * (2 * QT<Q>::kBlockBytes));
    }
    c.qoff = 16 + 32 * g;
    c.hout = hout;
    c.yout = yout;
    c.sorted = sorted;
    c.iexp = iexp;
    c.oexp = oexp;
    c.hdr = hdr;
    c.k = k;
    c.P = P;
    c.shared = shared;
    c.steps = K / BK;
    c.rows = rows;
    c.rb = rb;
    c.ct = ct;
    c.N = N;
    // only the row groups that hold rows of this tile run (an expert's last,
    // partial tile of a skewed batch is often far below BM rows)
    const int mi = (rows + 15) / 16;
    if (kMaxMI >= 8 && mi > 4) tile2_run<Q, GU, kMaxMI>(sm, c);
    else if (mi > 2) tile2_run<Q, GU, 4>(sm, c);
    else if (mi > 1) tile2_run<Q, GU, 2>(sm, c);
    else tile2_run<Q, GU, 1>(sm, c);
}

template <int Q, bool GU>
void launch2(const FwdArgs &a, const uint8_t *wa, const uint8_t *wb, const _Float16 *ain,
             _Float16 *hout, float *yout, int K, int N, int shared, const int32_t *iexp,
             int32_t *oexp, hipStream_t s) {
    const int col_tiles = GU ? N / 128 : N / BN;
    // routed: at most one partial tile per expert
    const int row_tiles = shared ? (a.T + BM - 1) / BM
                                 : std::min(a.L.max_tiles, (a.P + BM - 1) / BM + a.d.n_experts);
    const int nblk = (row_tiles + 7) / 8 * 8 * col_tiles;   // eight XCDs x whole row tiles
    gemm2_kernel<Q, GU><<<nblk, kThreads, 0, s>>>(
        wa, wb, (const int4 *)(a.ws + a.L.tiles), (WsHeader *)a.ws, a.sorted, ain, hout, yout,
        K, N, a.d.top_k, a.P, col_tiles, row_tiles, shared, shared ? a.T : 0, iexp, oexp);
}

}  // namespace

// One launch of format q (run-time) on the given matrices.
template <bool GU>
void launch2_q(int q, const FwdArgs &a, const uint8_t *wa, const uint8_t *wb,
               const _Float16 *ain, _Float16 *hout, float *yout, int K, int N, int shared,
               const int32_t *iexp, int32_t *oexp, hipStream_t s) {
    if (q == FW_Q4_0)
        launch2<FW_Q4_0, GU>(a, wa, wb, ain, hout, yout, K, N, shared, iexp, oexp, s);
    else if (q == FW_Q4_K)
        launch2<FW_Q4_K, GU>(a, wa, wb, ain, hout, yout, K, N, shared, iexp, oexp, s);
    else
        launch2<FW_Q8_0, GU>(a, wa, wb, ain, hout, yout, K, N, shared, iexp, oexp, s);
}

hipError_t launch_gemm2_gate_up(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const _Float16 *x = (const _Float16 *)(a.ws + a.L.x16);
    _Float16 *h = (_Float16 *)(a.ws + a.L.h);
    const int32_t *xe = (const int32_t *)(a.ws + a.L.xe);
    int32_t *he = (int32_t *)(a.ws + a.L.he);
    launch2_q<true>(d.expert_q, a, a.wg, a.wu, x, h, nullptr, d.hidden, d.ffn, 0, xe, he, s);
    if (d.shared_ffn > 0)
        launch2_q<true>(d.shared_q, a, a.sg, a.su, x, h + (size_t)a.P * d.ffn, nullptr, d.hidden,
                        d.shared_ffn, 1, xe, he + a.P, s);
    return hipGetLastError();
}

hipError_t launch_gemm2_down(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const _Float16 *h = (const _Float16 *)(a.ws + a.L.h);
    float *y = (float *)(a.ws + a.L.y);
    const int32_t *he = (const int32_t *)(a.ws + a.L.he);
    launch2_q<false>(d.expert_q, a, a.wd, nullptr, h, nullptr, y, d.ffn, d.hidden, 0, he,
                     nullptr, s);
    if (d.shared_ffn > 0)
        launch2_q<false>(d.shared_q, a, a.sd, nullptr, h + (size_t)a.P * d.ffn, nullptr,
                         y + (size_t)a.P * d.hidden, d.shared_ffn, d.hidden, 1, he + a.P,
                         nullptr, s);
    return hipGetLastError();
}

}  // namespace fw
