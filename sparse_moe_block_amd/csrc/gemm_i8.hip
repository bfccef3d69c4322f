// Forward with int8 expert activations on Q8_0 / Q4_0 experts (the pages'
// MMQ path: prompt processing's routed experts on block-table MMQ kernels,
// Flyweight 0.2.0 wheel METADATA, "Runtime controls"; activations quantised
// to int8 for them, "Image generation"): the staging of x as int8 blocks and
// the grouped expert GEMMs on the int8 MFMA.
//
// Quantisation (GGUF's Q8_1-style block of 32): d = fp32(max |v| / 127),
// codes round(fp32(v / d)), halves away from zero; d stays fp32.
//
// The contraction.  GGUF scales are per 32-element block of both operands, so
// one v_mfma_i32_32x32x32_i8 covers exactly one block: its K of 32 is the
// block.  Its exact int32 dot products S then take the block's two scales:
// y += (d_x d_w) S, a conversion, a product and an fma per output and block
// on the VALU -- the part that bounds this kernel (48 VALU instructions per
// 32-cycle int8 MFMA).  A lane's 16 outputs share its weight row (one d_w)
// and span 16 token rows, whose d_x it reads from LDS as four 16-byte runs
// (the step's activation scales sit there block-major).  Forming the d_x d_w
// tile on the matrix cores instead (an fp32 outer-product MFMA) saves the
// products but makes every tile's scaling wait for a second MFMA; Q8_0 does
// that all the same, its register budget having no room for the d_x runs.
//
// Weights reach the MFMA as stored: Q8_0 codes are int8 already; Q4_0 codes q
// become the int8 16 (q - 8) = (q << 4) ^ 0x80 (low nibble) or (q & 0xF0) ^
// 0x80 (high nibble), with d / 16 as the scale (exact).
//
// Tiles: 128 rows of one expert's pairs times 256 weight rows; eight
// wavefronts (two per SIMD), each all 128 token rows x 32 weight rows (one
// 32-column group; the accumulators are 64 VGPRs).  Gate/up: wavefronts 0..3
// hold gate features 128 ct + 32 w + n and wavefronts 4..7 the up features of
// the same 128; the up wavefronts hand their sums to the gate wavefronts
// through LDS at the end.  K advances 128 (four blocks) per step; a step's
// activation codes (128 x 128 bytes) and scales, and its weight blocks
// (256 rows x 4 blocks, as the 16-byte pieces that cover them) move HBM/L2
// -> LDS by DMA into one of two buffer sets while the other is used.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "stages.h"

namespace fw {
namespace {

constexpr int IBM = kGemmBM;          // token rows per tile
constexpr int IBN = 256;              // weight rows per tile
constexpr int IKS = 128;              // k per step (four blocks)
constexpr int INW = 8;                // wavefronts per workgroup
constexpr int IThreads = 64 * INW;
constexpr int kIAChunks = IBM * IKS / 16;   // 16-byte chunks of a step's activation codes
static_assert(IBM == 128 && kIAChunks == 2 * IThreads, "tile shape");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// Weight layout per format: bytes per block, 16-byte pieces per row and step
// (the smallest run of aligned pieces covering four blocks: they start at byte
// 0 of a piece on even steps and at byte 8 on odd ones), DMA instructions per
// thread for them (the last one padded with repeats of a valid piece).
constexpr int kIMaxWDma = 5;   // weight DMA instructions per thread and step, at most
template <int Q> struct I8W {
    static constexpr int kBlock = Q == FW_Q8_0 ? 34 : 18;
    static constexpr int kPieces = Q == FW_Q8_0 ? 9 : 5;
    static constexpr int kDma = (IBN * kPieces + IThreads - 1) / IThreads;
};

// int8 code of v for the block scale d > 0: round(v / d), halves away from
// zero, the division correctly rounded (HIP's fp32 division), within +-127.
__device__ __forceinline__ int q8_code(float v, float d) {
    return (int)fminf(fmaxf(roundf(v / d), -127.0f), 127.0f);
}

// One wavefront stages token row t as int8 blocks: each lane whole blocks
// (codes in k order to x8, d to xs).  A non-finite value sets
// FW_STATUS_RANGE (its block is stored as zeros).
__device__ __forceinline__ void stage_x_row_i8(const void *__restrict__ x, int act_bf16, int H,
                                               int t, int8_t *__restrict__ x8,
                                               float *__restrict__ xs,
                                               WsHeader *__restrict__ hdr) {
    const int lane = threadIdx.x % kWave, nb = H / 32;
    bool bad = false;
    for (int b = lane; b < nb; b += kWave) {
        float v[32];
        load_x_block(x, act_bf16, H, t, b, v);
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
        const bool nf = m >= 0x7F800000u;
        bad |= nf;
        const float d = nf ? 0.0f : __uint_as_float(m) / 127.0f;
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w |= (uint32_t)(d == 0.0f ? 0 : q8_code(v[4 * q + j], d) & 0xFF) << (8 * j);
            o[q] = w;
        }
        uint4 *dst = (uint4 *)(x8 + (size_t)t * H + 32 * b);
        dst[0] = uint4{o[0], o[1], o[2], o[3]};
        dst[1] = uint4{o[4], o[5], o[6], o[7]};
        xs[(size_t)t * nb + b] = d;
    }
    if (bad) atomicOr(&hdr->status, FW_STATUS_RANGE);
}

// Block 0: the schedule (active experts, 128-row tiles); the other blocks:
// one wavefront per token row, staged as int8.
__global__ __launch_bounds__(kPrepThreads) void prepare_i8_kernel(
    const int32_t *__restrict__ offsets, int E, int P, const void *__restrict__ x, int act_bf16,
    int H, int T, int max_tiles, int4 *__restrict__ active, int4 *__restrict__ tiles,
    int8_t *__restrict__ x8, float *__restrict__ xs, int *__restrict__ split_cnt,
    WsHeader *__restrict__ hdr) {
    if (blockIdx.x == 0) {
        build_schedule(offsets, E, P, IBM, max_tiles, active, tiles, split_cnt, hdr,
                       kCostI8);
        return;
    }
    const int t = (blockIdx.x - 1) * (kPrepThreads / kWave) + wave_id();
    if (t >= T) return;
    stage_x_row_i8(x, act_bf16, H, t, x8, xs, hdr);
}

// The lane's 16 codes (k 16 g .. 16 g + 15 of block b) of its weight row and
// the block's scale, from the row's pieces in LDS (row: its first piece;
// first: the step's byte offset in it, 0 or 8).  Q4_0 codes come out as
// 16 (q - 8) and the scale as d / 16.
template <int Q, int first, int b>
__device__ __forceinline__ void weight_frag(const uint8_t *row, int g, v4i &w, float &d) {
    constexpr int BB = I8W<Q>::kBlock;
    constexpr int hd = first + BB * b;   // the block's fp16 scale
    const uint32_t dw = *(const uint32_t *)(row + (hd & ~3));
    d = (float)__builtin_bit_cast(_Float16, (uint16_t)((hd & 2) ? dw >> 16 : dw & 0xFFFFu));
    // code bytes from hd + 2 (Q8_0: + 16 g)
    const uint8_t *c = row + hd + 2 + (Q == FW_Q8_0 ? 16 * g : 0);
    uint32_t r[4];
    if constexpr (((hd + 2) & 3) == 0) {
        const uint32_t *p = (const uint32_t *)c;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = p[i];
    } else {   // 2 mod 4: five dwords, shifted by two bytes
        const uint32_t *p = (const uint32_t *)(c - 2);
        uint32_t s[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) s[i] = p[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbyte(s[i + 1], s[i], 2);
    }
    if constexpr (Q == FW_Q4_0) {
        // elements 16 g .. 16 g + 15: low nibbles (g = 0) or high nibbles (g = 1)
        const uint32_t sh = g ? 0u : 4u;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = ((r[i] << sh) & 0xF0F0F0F0u) ^ 0x80808080u;
        d *= 0.0625f;
    }
    w = v4i{(int)r[0], (int)r[1], (int)r[2], (int)r[3]};
}

// One (row tile, column tile) of one expert (or of the shared expert).
//  GU:  A = x8 rows (routed: the tokens of the sorted pairs); weights = 128
//       gate + 128 up features; writes h = int8(SiLU(g) * u) (codes to h8,
//       one fp32 scale per row and 32 features to hsc), row stride N;
//  !GU: A = h8 rows (stride K); weights = 256 outputs; writes y (fp32).
template <int Q, bool GU>
__global__ __launch_bounds__(IThreads, 1) void gemm_i8_kernel(
    const uint8_t *__restrict__ wa, const uint8_t *__restrict__ wb,
    const int4 *__restrict__ tiles, WsHeader *__restrict__ hdr,
    const int32_t *__restrict__ sorted, const int8_t *__restrict__ a8,
    const float *__restrict__ asc, int8_t *__restrict__ h8, float *__restrict__ hsc,
    float *__restrict__ yout, int K, int N, int k, int P, int col_tiles, int n_row_tiles_max,
    int shared, int shared_rows) {
    constexpr int BB = I8W<Q>::kBlock, PX = I8W<Q>::kPieces, WD = I8W<Q>::kDma;
    // two buffer sets, each its own array (the compiler tells a pending DMA
    // into one from reads of the other only when they are distinct objects)
    __shared__ uint4 A0[kIAChunks], A1[kIAChunks];
    __shared__ float AS0[4 * IBM], AS1[4 * IBM];   // the step's block scales, [block][row]
    static_assert(WD <= kIMaxWDma, "weight pieces");
    __shared__ uint4 B0[WD * IThreads], B1[WD * IThreads];
    auto Abuf = [&](int buf) { return buf ? A1 : A0; };
    auto ASbuf = [&](int buf) { return buf ? AS1 : AS0; };
    auto Bbuf = [&](int buf) { return buf ? B1 : B0; };
    // XCD-aware order (the tiles of one expert are consecutive)
    int ct;
    const int rt = xcd_row_tile(hdr, col_tiles, n_row_tiles_max, shared,
                                (shared_rows + IBM - 1) / IBM, ct);
    if (rt < 0) return;
    int expert = 0, rb = 0, rows = 0;
    if (shared) {
        rb = rt * IBM;
        rows = min(IBM, shared_rows - rb);
    } else {
        const int4 tl = ld_const(tiles + rt);   // (expert, first row, rows)
        expert = tl.x;
        rb = tl.y;
        rows = tl.z;
    }
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int n = lane & 31, g = lane >> 5;
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
    // activation codes: slot s is position s % 8 of tile row s / 8 and holds
    // its chunk (s % 8) ^ (row % 8), so that the lanes reading one chunk of 8
    // consecutive rows hit distinct banks
    uint32_t aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int s = i * IThreads + tid, r = s / 8, c = (s % 8) ^ (r % 8);
        aoff[i] = (uint32_t)src_row(r) * (uint32_t)K + 16u * c;
    }
    // activation scales: slot tid is block tid / 128 of the step, tile row
    // tid % 128
    const uint32_t asoff = ((uint32_t)src_row(tid % IBM) * (uint32_t)(K / 32) + tid / IBM) * 4u;
    // weight rows: LDS row Rl is matrix row wrow(Rl) of the expert (gate/up:
    // rows 128 .. 255 are the up matrix's)
    const size_t rowbytes = (size_t)(K / 32) * BB;
    const uint8_t *gbase = wa + (size_t)expert * N * rowbytes;
    const uint8_t *ubase = (GU ? wb : wa) + (size_t)expert * N * rowbytes;
    // weight pieces: slot p is piece p % PX of LDS row p / PX; slots past the
    // tile's 256 PX pieces repeat its last piece
    // (a fixed size: a local array whose size depends on Q, captured by the
    // lambdas below, breaks their host-side instantiation)
    uint32_t woff[kIMaxWDma];
    uint32_t wup = 0;   // bit i: slot i reads the up matrix
#pragma unroll
    for (int i = 0; i < WD; ++i) {
        const int p = min(i * IThreads + tid, IBN * PX - 1), Rl = p / PX, j = p % PX;
        const int row = GU ? ct * 128 + (Rl & 127) : ct * 256 + Rl;
        woff[i] = (uint32_t)((size_t)row * rowbytes) + 16u * j;
        if (GU && Rl >= 128) wup |= 1u << i;
    }

    // The main loop for MI 32-row groups (the groups that hold rows of the
    // tile).  MI is a template parameter so that the loop body has no branch:
    // the compiler would otherwise sink a step's MFMAs past the DMA wait.
    auto run = [&]<int MI>() {
    auto dma = [&](int buf, int st, int part) {
        if (part == 0) {
            const uint32_t ka = (uint32_t)st * IKS, ks = (uint32_t)st * 16u;
#pragma unroll
            for (int i = 0; i < (MI + 1) / 2; ++i)   // rows 64 i .. 64 i + 63
                __builtin_amdgcn_global_load_lds((const uint8_t *)a8 + (aoff[i] + ka),
                                                 (lds_void *)(&Abuf(buf)[i * IThreads + 64 * wave]),
                                                 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const uint8_t *)asc + (asoff + ks),
                                             (lds_void *)(&ASbuf(buf)[64 * wave]), 4, 0, 0);
        } else {
            // step st starts at byte 4 BB st of the rows, in its piece at 0 or 8
            const uint32_t kb = (uint32_t)(st * 4 * BB) & ~15u;
#pragma unroll
            for (int i = 0; i < WD; ++i)
                __builtin_amdgcn_global_load_lds(((wup >> i) & 1 ? ubase : gbase) + (woff[i] + kb),
                                                 (lds_void *)(&Bbuf(buf)[i * IThreads + 64 * wave]),
                                                 16, 0, 0);
        }
    };
    // everything issued so far has landed and every wavefront is here
    auto sync = [&]() {
        __builtin_amdgcn_s_waitcnt(7 << 4);   // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    f16v acc[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
    const v16i izero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const f16v fzero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                        0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int steps = K / IKS;
    const int Rw = 32 * wave + n;   // the lane's LDS weight row
    // how a block tile's scales d_x d_w are formed (see FW_I8_BLOCK)
    constexpr bool kVecScale = Q == FW_Q4_0;

    // one step from buffer set BUF (first piece byte 8 BUF); pf(b) issues the
    // next step's DMA after block b's MFMAs
    auto step = [&](auto bufc, auto &&pf) {
        constexpr int BUF = decltype(bufc)::value;
        const uint8_t *wrow = (const uint8_t *)Bbuf(BUF) + Rw * (16 * PX);
        const uint4 *abuf = Abuf(BUF);
        const float *as = ASbuf(BUF);
        v4i a[2][MI], w[2];
        float dw[2];
        float dxl[2][MI], dwl[2];   // Q8_0: the outer-product MFMA's operands
        auto load = [&](auto xc, auto bc) {
            constexpr int X = decltype(xc)::value, b = decltype(bc)::value;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int r = 32 * mi + n;
                a[X][mi] = __builtin_bit_cast(v4i, abuf[8 * r + ((2 * b + g) ^ (r % 8))]);
                if constexpr (!kVecScale) {
                    const float d = as[IBM * b + r];
                    dxl[X][mi] = g ? 0.0f : d;
                }
            }
            weight_frag<Q, 8 * BUF, b>(wrow, g, w[X], dw[X]);
            if constexpr (!kVecScale) dwl[X] = g ? 0.0f : dw[X];
        };
        // d_x of the lane's 16 output rows of group mi, block b: rows
        // 32 mi + 8 j + 4 g + i (output element 4 j + i), four runs of 4
        auto scales_x = [&](int b, int mi, float4 *dx) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dx[j] = *(const float4 *)&as[IBM * b + 32 * mi + 8 * j + 4 * g];
        };
        load(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    // Block B: the next block's operands are read first; then row group mi's
    // MFMAs (and d_x reads) are issued ahead of the scaling of group mi - 1's
    // sums, so at most two groups' sums and scales are live.
    //  - Q4_0: d_x d_w on the VALU, d_x read a group ahead;
    //  - Q8_0: its wider weight reads leave too few registers for that (the
    //    VALU form spilled), so the d_x d_w tile comes from an fp32
    //    outer-product MFMA (v_mfma_f32_32x32x2_f32, the second k term zero:
    //    each lane supplies its row's d_x and its weight row's d_w).
#define FW_I8_BLOCK(B)                                                                        \
    {                                                                                         \
        constexpr int X = (B) & 1;                                                            \
        if constexpr ((B) < 3)                                                                \
            load(std::integral_constant<int, X ^ 1>{}, std::integral_constant<int, (B) + 1>{}); \
        v16i s[2];                                                                            \
        float4 dx[2][4];                                                                      \
        f16v c[2];                                                                            \
        _Pragma("unroll") for (int mi = 0; mi <= MI; ++mi) {                                  \
            if (mi < MI) {                                                                    \
                s[mi & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[X][mi], w[X], izero, 0,   \
                                                                  0, 0);                      \
                if constexpr (kVecScale) {                                                    \
                    scales_x((B), mi, dx[mi & 1]);                                            \
                } else {                                                                      \
                    c[mi & 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(dxl[X][mi], dwl[X], fzero, \
                                                                     0, 0, 0);                \
                }                                                                             \
            }                                                                                 \
            if (mi > 0) {                                                                     \
                const int p = (mi - 1) & 1;                                                   \
                _Pragma("unroll") for (int v = 0; v < 16; ++v) {                              \
                    float sc;                                                                 \
                    if constexpr (kVecScale) {                                                \
                        const float4 q = dx[p][v >> 2];                                       \
                        sc = ((v & 3) == 0 ? q.x : (v & 3) == 1 ? q.y                         \
                                                 : (v & 3) == 2 ? q.z : q.w) * dw[X];         \
                    } else {                                                                  \
                        sc = c[p][v];                                                         \
                    }                                                                         \
                    acc[mi - 1][v] = __builtin_fmaf((float)s[p][v], sc, acc[mi - 1][v]);      \
                }                                                                             \
            }                                                                                 \
            __builtin_amdgcn_sched_barrier(0);                                                \
        }                                                                                     \
        pf(B);                                                                                \
        __builtin_amdgcn_sched_barrier(0);                                                    \
    }
        FW_I8_BLOCK(0)
        FW_I8_BLOCK(1)
        FW_I8_BLOCK(2)
        FW_I8_BLOCK(3)
#undef FW_I8_BLOCK
    };
    // Step st uses buffer set st % 2 and loads step st + 1 into the other,
    // which every wavefront finished reading before the sync that ended step
    // st - 1.  K is a multiple of 256, so the steps come in pairs; after the
    // last pair the prefetch repeats the last step's addresses (no DMA reaches
    // past the rows).
    dma(0, 0, 0);
    dma(0, 0, 1);
    sync();
    for (int st = 0; st < steps; st += 2) {
        step(std::integral_constant<int, 0>{}, [&](int b) { if (b < 2) dma(1, st + 1, b); });
        sync();
        const int nx = min(st + 2, steps - 1);
        step(std::integral_constant<int, 1>{}, [&](int b) { if (b < 2) dma(0, nx, b); });
        sync();
    }

    // ---- epilogue: acc[mi][v] is tile row 32 mi + 8 (v / 4) + 4 g + v % 4,
    // LDS weight row 32 wave + n ----
    bool range = false;
    if constexpr (GU) {
        // the up wavefronts (4..7) hand their sums to the gate wavefronts
        // (0..3) with the same features through A0 (its last DMA has landed),
        // one 32-row group at a time: 4 wavefronts x 16 values x 64 lanes
        float *xch = (float *)A0;
        const int f0 = 128 * ct + 32 * (wave & 3);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            if (wave >= 4) {
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    xch[((wave - 4) * 16 + v) * 64 + lane] = acc[mi][v];
            }
            __syncthreads();
            if (wave < 4) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 32 * mi + 8 * (v >> 2) + 4 * g + (v & 3);
                    const float gv = acc[mi][v], up = xch[(wave * 16 + v) * 64 + lane];
                    const float av = gv / (1.0f + __expf(-gv)) * up;
                    // the row's 32 features are the 32 lanes of this half
                    uint32_t m = __float_as_uint(av) & 0x7FFFFFFFu;
#pragma unroll
                    for (int o = 1; o < 32; o <<= 1)
                        m = max(m, (uint32_t)__shfl_xor((int)m, o, 32));
                    if (row < rows) {
                        const bool nf = m >= 0x7F800000u;
                        range |= nf;
                        const float d = nf ? 0.0f : __uint_as_float(m) / 127.0f;
                        const size_t hr = (size_t)(rb + row);
                        h8[hr * N + f0 + n] = (int8_t)(d == 0.0f ? 0 : q8_code(av, d));
                        if (n == 0) hsc[hr * (N / 32) + f0 / 32] = d;
                    }
                }
            }
            __syncthreads();
        }
    } else {
        float *yrow = yout + (size_t)ct * 256 + 32 * wave + n;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 32 * mi + 8 * (v >> 2) + 4 * g + (v & 3);
                if (row < rows) yrow[(size_t)(rb + row) * N] = acc[mi][v];
            }
    }
    if (range) atomicOr(&hdr->status, FW_STATUS_RANGE);
    };
    const int mi = (rows + 31) / 32;
    if (mi > 3) run.template operator()<4>();
    else if (mi > 2) run.template operator()<3>();
    else if (mi > 1) run.template operator()<2>();
    else run.template operator()<1>();
}

// The int8 areas inside the fp16 staging areas of the workspace: x8 [T][H]
// then its scales [T][H/32] (fp32); h8 [P][F] then [T][Fs], then their scales.
struct I8Areas {
    int8_t *x8, *h8;
    float *xs, *hs;
};
I8Areas i8_areas(const FwdArgs &a) {
    I8Areas m;
    m.x8 = (int8_t *)(a.ws + a.L.x16);
    m.xs = (float *)(m.x8 + (size_t)a.T * a.d.hidden);
    m.h8 = (int8_t *)(a.ws + a.L.h);
    m.hs = (float *)(m.h8 + (size_t)a.P * a.d.ffn + (size_t)a.T * a.d.shared_ffn);
    return m;
}

template <bool GU>
void launch_i8(const FwdArgs &a, int q, const uint8_t *wa, const uint8_t *wb, const int8_t *a8,
               const float *asc, int8_t *h8, float *hsc, float *yout, int K, int N, int shared,
               hipStream_t s) {
    const int col_tiles = GU ? N / 128 : N / 256;
    const int row_tiles = shared ? (a.T + IBM - 1) / IBM
                                 : gemm_row_tiles(a.P, a.d.n_experts, IBM, a.L.max_tiles);
    const int nblk = (row_tiles + 7) / 8 * 8 * col_tiles;   // eight XCDs x whole row tiles
    if (q == FW_Q4_0)
        gemm_i8_kernel<FW_Q4_0, GU><<<nblk, IThreads, 0, s>>>(
            wa, wb, (const int4 *)(a.ws + a.L.tiles), (WsHeader *)a.ws, a.sorted, a8, asc, h8,
            hsc, yout, K, N, a.d.top_k, a.P, col_tiles, row_tiles, shared, shared ? a.T : 0);
    else
        gemm_i8_kernel<FW_Q8_0, GU><<<nblk, IThreads, 0, s>>>(
            wa, wb, (const int4 *)(a.ws + a.L.tiles), (WsHeader *)a.ws, a.sorted, a8, asc, h8,
            hsc, yout, K, N, a.d.top_k, a.P, col_tiles, row_tiles, shared, shared ? a.T : 0);
}

}  // namespace

hipError_t launch_prepare_i8(const FwdArgs &a, hipStream_t s) {
    const I8Areas m = i8_areas(a);
    constexpr int rows_per_block = kPrepThreads / kWave;   // one wavefront per token row
    prepare_i8_kernel<<<1 + (a.T + rows_per_block - 1) / rows_per_block, kPrepThreads, 0, s>>>(
        a.offsets, a.d.n_experts, a.P, a.x, a.d.act_dtype == FW_BF16, a.d.hidden, a.T,
        a.L.max_tiles, (int4 *)(a.ws + a.L.active), (int4 *)(a.ws + a.L.tiles), m.x8, m.xs,
        (int *)(a.ws + a.L.split_cnt), (WsHeader *)a.ws);
    return hipGetLastError();
}

hipError_t launch_gemm_i8_gate_up(const FwdArgs &a, hipEvent_t routed_done, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const I8Areas m = i8_areas(a);
    const size_t hr = (size_t)a.P * d.ffn;   // the shared expert's h rows start here
    launch_i8<true>(a, d.expert_q, a.wg, a.wu, m.x8, m.xs, m.h8, m.hs, nullptr, d.hidden, d.ffn,
                    0, s);
    if (routed_done) (void)hipEventRecord(routed_done, s);
    if (d.shared_ffn > 0)
        launch_i8<true>(a, d.shared_q, a.sg, a.su, m.x8, m.xs, m.h8 + hr, m.hs + hr / 32,
                        nullptr, d.hidden, d.shared_ffn, 1, s);
    return hipGetLastError();
}

hipError_t launch_gemm_i8_down(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const I8Areas m = i8_areas(a);
    const size_t hr = (size_t)a.P * d.ffn;
    float *y = (float *)(a.ws + a.L.y);
    launch_i8<false>(a, d.expert_q, a.wd, nullptr, m.h8, m.hs, nullptr, nullptr, y, d.ffn,
                     d.hidden, 0, s);
    if (d.shared_ffn > 0)
        launch_i8<false>(a, d.shared_q, a.sd, nullptr, m.h8 + hr, m.hs + hr / 32, nullptr,
                         nullptr, y + (size_t)a.P * d.hidden, d.shared_ffn, d.hidden, 1, s);
    return hipGetLastError();
}

}  // namespace fw
