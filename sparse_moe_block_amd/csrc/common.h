// Internal declarations of the gfx950 MoE library: workspace layout, GGUF block
// decoding in registers, and the kernel launchers the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fwmoe.h"

namespace fw {

constexpr int kWave = 64;
constexpr int kMaxDevices = 64;   // per-device caches of device properties
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;
constexpr int kUnit = 256;        // elements per 16-byte-aligned run of 8 blocks
constexpr int kGemvTokens = 2;    // token rows a GEMV work item carries
constexpr int kGemmBM = 128;      // token rows per tile of the int8 GEMM
// Token rows per tile of the fp16 grouped GEMM: five 32-row groups for Q4_0
// experts, four for the other formats (whose fragments need more registers).
// An expert whose segment has at most this many rows is one tile.
constexpr int gemm_tile_rows(int q) { return q == FW_Q4_0 ? 160 : 128; }
// Bound on the row tiles of a routed GEMM (at most one partial tile per
// expert), and the row tiles each XCD's share of the launch has room for:
// a launch holds 8 * xcd_tile_cap rows of column tiles of workgroups.
__host__ __device__ constexpr int gemm_row_tiles(int P, int E, int tile_rows, int max_tiles) {
    return (P + tile_rows - 1) / tile_rows + E < max_tiles ? (P + tile_rows - 1) / tile_rows + E
                                                           : max_tiles;
}
__host__ __device__ constexpr int xcd_tile_cap(int P, int E, int tile_rows, int max_tiles) {
    return (gemm_row_tiles(P, E, tile_rows, max_tiles) + 7) / 8;
}
// Work estimate of a grouped-GEMM row tile by kernel, for splitting the tile
// list among the XCDs: a fixed part for an expert's first tile and for each
// later tile of the expert, and a part per 32-row MFMA group.  Measured on
// Zipf-routed prefill: the eight-wave fp16 and the int8 kernels run faster
// with ranges of equal estimated work (a one-group tile costing about half a
// four-group one, as timed on the DeepSeek-shaped layer; for Q4_0's 160-row
// tiles a larger fixed part, (12, 12, 2) against (3, 3, 2): gate/up 170 ->
// 160 us, while Q4_K and MXFP4 were 4-5 % slower with it); the four-wave
// fp16 and the block-scaled kernels with ranges of equal tile counts -- by
// work their gate/up launches were 4-8 % slower, and slower still when an
// expert's later tiles counted less.
struct TileCost {
    int first, rep, group;
};
constexpr TileCost kCostF16Q4{12, 12, 2};  // fp16, Q4_0 (160-row tiles)
constexpr TileCost kCostF16{3, 3, 2};      // fp16, eight-wave workgroups (Q4_K, MXFP4)
constexpr TileCost kCostF16W4{1, 1, 0};    // fp16, four-wave workgroups (Q8_0, Q6_K): counts
constexpr TileCost kCostMx8{1, 1, 0};      // block-scaled MFMA (MXFP8 activations): counts
constexpr TileCost kCostI8{3, 3, 2};       // int8 MFMA
constexpr TileCost gemm_tile_cost(int q) {
    return q == FW_Q4_0                   ? kCostF16Q4
           : q == FW_Q8_0 || q == FW_Q6_K ? kCostF16W4
                                          : kCostF16;
}
// AUTO: the GEMV family while the routed pairs average at most this many rows
// per expert (T * k <= 2 E), the grouped GEMM above.  Measured crossovers, in
// rows per expert: the hidden-4096 / 64-expert top-4 layer between 2 and 3
// (Q8_0 and Q4_0, uniform and Zipf(1.3) routing), the Qwen3-shaped layer
// between 1.5 and 2 (a tie at 2), the DeepSeek-shaped layer between 1.5 and 2.
constexpr int kGemvMaxRowsPerExpert = 2;
// router logits: the 16-token-tile kernel up to this many tokens
constexpr int kLogitsTileMaxT = 64;
// GEMV split-K: at most this many (row chunk, weight tile) pairs are split,
// into at most kSplitSlicesMax reduction slices each
constexpr int kSplitTiles = 1024;
constexpr int kSplitSlicesMax = 8;

// Per-token scaling of the fp16 operands.  Each token row of x is staged as
// x * 2^e, e chosen so that its largest magnitude lands in
// [2^(kXExp-1), 2^kXExp): any finite row then uses fp16's normal range the
// same way, whatever its own scale.  The gate/up accumulators are multiplied
// by 2^-e (exact) before SwiGLU, and the SwiGLU output h is stored as
// h * 2^(2e) -- g and u scale with x, so that keeps h near the range of a
// unit-scale row -- and the down projection's accumulators are multiplied by
// 2^-2e.  kXExp = 5 leaves h about 16x of headroom below fp16's 65504 on
// the workloads' weights; larger values set FW_STATUS_RANGE.
constexpr int kXExp = 5;
// Largest fp16 scale bits (magnitude) whose 16x-scaled extreme code stays
// within fp16 in the grouped GEMM's dequantised weights: Q4_0 16 * 8 * d
// <= 65504 (d <= 511.75), Q8_0 16 * 128 * d <= 65504 (d <= 31.984375).
constexpr uint32_t kQ4DMaxBits = 0x5FFFu;
constexpr uint32_t kQ8DMaxBits = 0x4FFFu;

// First 256 bytes of every workspace.
struct WsHeader {
    int32_t status;     // sticky FW_STATUS_* bits
    int32_t n_active;   // experts with at least one routed pair
    int32_t n_tiles;    // row tiles of the routed experts (GEMM tiles or GEMV chunks)
    // GEMM tiles: XCD x runs row tiles [xcd_first[x], xcd_first[x + 1])
    int32_t xcd_first[9];
    int32_t reserved[52];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

// Byte offsets of the per-call scratch areas inside the workspace.
struct WsLayout {
    size_t active;   // int4 [E + 1]              (expert, first row, rows) per active expert
    size_t tiles;    // int4 [max_tiles]          (expert, first row, rows) per row tile
    size_t x16;      // f16  [T][H]               x in pair order
    size_t h;        // f16  [P][F] then [T][Fs]  SiLU(g)*u in pair order
    size_t y;        // f32  [P][H] then [T][H]   per-pair expert outputs
    size_t split_cnt;   // int [kSplitTiles]      split-K arrival counters
    size_t split_part;  // f32 [kSplitTiles * kSplitSlicesMax][2 * kGemvTokens][64] partials
    size_t xe;       // int  [T]                  power-of-two exponent x16 row t is scaled by
    size_t he;       // int  [P + T]              the same for h rows (2 xe of the row's token)
    size_t xsum;     // f32  [T][H/32]            32-element block sums of x16 (Q4_K GEMV)
    size_t hsum;     // f32  [P][F/32] then [T][Fs/32]   block sums of h (Q4_K GEMV)
    size_t perm;     // int [E][nb + 1]              multi-block permutation: per-block
                     //                              counts, then their prefix; totals
    size_t total;
    int max_tiles;
};
WsLayout ws_layout(const fw_moe_desc &d, int T);

// ---------------------------------------------------------------------------
// GGUF blocks in registers.  A "unit" is 8 consecutive blocks (256 elements):
// 144 bytes for Q4_0, 272 for Q8_0, both multiples of 16, so every unit of a
// row whose length is a multiple of 256 starts 16-byte aligned and loads as
// whole dwordx4s.  Block b of a unit starts at byte 18b (34b); even blocks
// start dword-aligned (their codes are 2 bytes off), odd blocks start 2 bytes
// off (their codes are dword-aligned).
template <int Q> struct QT;
template <> struct QT<FW_Q4_0> {
    static constexpr int kBlockBytes = 18, kUnitBytes = 144, kUnitX4 = 9;
    static constexpr size_t row_bytes(int K) { return (size_t)(K / 32) * kBlockBytes; }
};
template <> struct QT<FW_Q8_0> {
    static constexpr int kBlockBytes = 34, kUnitBytes = 272, kUnitX4 = 17;
    static constexpr size_t row_bytes(int K) { return (size_t)(K / 32) * kBlockBytes; }
};
// Q4_K: a unit is one 256-element super-block (144 bytes; kBlockBytes is the
// per-32-element share used to size rows): [fp16 d][fp16 dmin][12 bytes of
// six-bit (scale, min) pairs][128 code bytes], group c of 64 elements in code
// bytes 32c .. 32c + 31 (low nibbles: sub-block 2c, high: 2c + 1).
template <> struct QT<FW_Q4_K> {
    static constexpr int kBlockBytes = 18, kUnitBytes = 144, kUnitX4 = 9;
    static constexpr size_t row_bytes(int K) { return (size_t)(K / 256) * kUnitBytes; }
};
// Q6_K: a unit is one 256-element super-block of 210 bytes, [128 bytes ql]
// [64 bytes qh][16 int8 scales][fp16 d]: half h (128 elements) uses ql bytes
// 64h .. 64h + 63 and qh bytes 32h .. 32h + 31; element 32k + l of the half
// takes the low (k < 2) or high (k >= 2) nibble of ql byte 64h + 32 (k % 2) + l
// and bits 2k, 2k + 1 of qh byte 32h + l as a six-bit code q; value
// d * scale_(e / 16) * (q - 32).  Units are 2-byte aligned only: a unit is
// staged as the 14 aligned 16-byte pieces that cover it (kUnitX4), at a
// per-row byte offset of 0 .. 14 into the first piece.
template <> struct QT<FW_Q6_K> {
    static constexpr int kUnitBytes = 210, kUnitX4 = 14;
    static constexpr size_t row_bytes(int K) { return (size_t)(K / 256) * kUnitBytes; }
};
// MXFP4 (MLX packing, group 32): a matrix of R rows is R x K/2 bytes of E2M1
// codes (element j in nibble j % 2 of byte j / 2) followed by R x K/32 E8M0
// scale bytes.  Rows here are code rows (row_bytes); a row's scales sit at
// the matrix base + R K/2 + row K/32.  A unit is the 128 code bytes of 256
// elements plus the 16-byte aligned piece holding its 8 scales (kUnitX4 = 9).
template <> struct QT<FW_MXFP4> {
    static constexpr int kUnitBytes = 128, kUnitX4 = 9;
    static constexpr size_t row_bytes(int K) { return (size_t)K / 2; }
};


// Uniform read of data no kernel writes while the reader runs (schedules,
// pair lists, staged activations): through the constant address space, which
// the compiler turns into a scalar load when the address is uniform.
__device__ __forceinline__ int ld_const(const int *p) {
    return *(const __attribute__((address_space(4))) int *)p;
}
__device__ __forceinline__ int4 ld_const(const int4 *p) {
    const int *q = (const int *)p;
    return int4{ld_const(q), ld_const(q + 1), ld_const(q + 2), ld_const(q + 3)};
}

// The row tile a grouped-GEMM workgroup runs (-1: none) and, in ct, its
// column tile.  Workgroup b runs on XCD b % 8; each XCD takes a contiguous
// range of row tiles, column tiles fastest: for the routed experts the
// schedule's ranges of about equal work (hdr->xcd_first, at most
// n_row_tiles_max / 8 rounded up tiles each, which the launch has room
// for), for the shared expert's n_shared tiles eighths.
__device__ __forceinline__ int xcd_row_tile(const WsHeader *hdr, int col_tiles,
                                            int n_row_tiles_max, int shared, int n_shared,
                                            int &ct) {
    const int xcd = blockIdx.x % 8, bi = blockIdx.x / 8;
    const int rl = bi / col_tiles;
    ct = bi % col_tiles;
    if (shared) {
        const int per = (n_shared + 7) / 8, rt = xcd * per + rl;
        return rl < per && rt < n_shared ? rt : -1;
    }
    const int n_rt = min(ld_const(&hdr->n_tiles), n_row_tiles_max);
    const int rt = ld_const(&hdr->xcd_first[xcd]) + rl;
    return rt < min(ld_const(&hdr->xcd_first[xcd + 1]), n_rt) ? rt : -1;
}

// The wavefront index inside the workgroup, as a value the compiler knows to
// be uniform across the wavefront (so loops over it stay in scalar registers).
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
    return (float)h;
}

__device__ __forceinline__ uint32_t funnel16(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_alignbyte(hi, lo, 2);   // bytes 2..5 of hi:lo
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }

// The code dwords of block B of a unit held as dwords w[] (4 for Q4_0, 8 for
// Q8_0, realigned), and its fp16 scale as fp32.
template <int Q, int B>
__device__ __forceinline__ float block_codes(const uint32_t *w, uint32_t *q) {
    if constexpr (Q == FW_Q4_0) {
        constexpr int base = (B / 2) * 9;   // dword index of the even block of the pair
        if constexpr (B % 2 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = funnel16(w[base + i], w[base + i + 1]);
            return half_bits_to_float(w[base] & 0xFFFFu);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = w[base + 5 + i];
            return half_bits_to_float(w[base + 4] >> 16);
        }
    } else {
        constexpr int base = (B / 2) * 17;
        if constexpr (B % 2 == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = funnel16(w[base + i], w[base + i + 1]);
            return half_bits_to_float(w[base] & 0xFFFFu);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = w[base + 9 + i];
            return half_bits_to_float(w[base + 8] >> 16);
        }
    }
}

// Pair order.  The 32 elements of a block are consumed as 16 fp16 pairs; pair
// 4m+j (m = 0..3) holds elements
//   j = 0: (4m, 4m+2)          j = 1: (16+4m, 16+4m+2)
//   j = 2: (4m+1, 4m+3)        j = 3: (16+4m+1, 16+4m+3)
// On the weight side pairs j = 1, 3 carry 16 * value, on the activation side
// value / 16 (exact scalings), so every pair product is unchanged.  This order
// lets a Q4_0 code dword become four pairs with one mask each: the low nibbles
// of bytes 0 and 2 sit at bits 0 and 16, their high nibbles at bits 4 and 20.
__device__ __forceinline__ int pair_pos(int i) {   // element i -> half index in its block
    const int hi = i >> 4, m = (i & 15) >> 2, j = i & 3;
    return 2 * (4 * m + (j & 1) * 2 + hi) + (j >> 1);
}

// Block B of a unit as 16 exact fp16 pairs (in pair order) times its scale d:
// value of element i = d * (pair value), pairs j = 1, 3 scaled by 16.
// The integer-to-fp16 step is the published "magic number" conversion: OR the
// code bits into the mantissa of an fp16 1024 (exponent 0x6400), then subtract
// the constant, all exact (Kim et al., "Who Says Elephants Can't Run: Bringing
// Large Scale MoE Models into Cloud Scale Production", arXiv 2211.10017, and
// the interleaved int4 -> fp16 conversion of NVIDIA FasterTransformer).  What
// is ours: the pair order below (one mask per pair, high nibbles kept in place
// as 16 q with the matching activations pre-scaled by 1/16), the v_perm form
// for Q8_0, and the block scale applied in one rounding.
//  Q4_0: (c & 0x000F000F) | 0x6400_6400 is the pair 1024 + q; minus 1032 gives
//        q - 8.  The high nibbles masked in place give 1024 + 16q; minus 1152
//        gives 16(q - 8).
//  Q8_0: c ^ 0x80808080 turns signed codes into q + 128; v_perm places two of
//        them under a 0x64 exponent byte: 1024 + 128 + q; minus 1152 gives q,
//        and for j = 1, 3 a fused 16x - 18432 gives 16q.  All exact in fp16.
// (c & m) | k in one v_and_or_b32.  gfx950's VOP3 encoding takes no literal
// constants, so the mask travels in an SGPR and the exponent bits in a VGPR
// set up once; left to itself the compiler splits the expression into a
// v_and and a v_or with literals.
__device__ __forceinline__ uint32_t and_or(uint32_t c, uint32_t m, uint32_t k) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(c), "s"(m), "v"(k));
    return r;
}

// The 16 exact fp16 pairs of one block from its realigned code dwords q[]
// (4 for Q4_0, 8 for Q8_0), in pair order.
template <int Q>
__device__ __forceinline__ void codes_to_pairs(const uint32_t *q, h2 *p, uint32_t magic) {
    const h2 k1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 k1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
    if constexpr (Q == FW_Q4_0) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t c = q[m], c8 = q[m] >> 8;
            p[4 * m + 0] = as_h2(and_or(c, 0x000F000Fu, magic)) - k1032;
            p[4 * m + 1] = as_h2(and_or(c, 0x00F000F0u, magic)) - k1152;
            p[4 * m + 2] = as_h2(and_or(c8, 0x000F000Fu, magic)) - k1032;
            p[4 * m + 3] = as_h2(and_or(c8, 0x00F000F0u, magic)) - k1152;
        }
    } else {
        const h2 k16 = {(_Float16)16.0f, (_Float16)16.0f};
        const h2 k18432 = {(_Float16)18432.0f, (_Float16)18432.0f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t lo = q[m] ^ 0x80808080u, hi = q[4 + m] ^ 0x80808080u;
            // byte selectors: 0..3 pick from the second operand, 4..7 from the first
            p[4 * m + 0] = as_h2(__builtin_amdgcn_perm(magic, lo, 0x04020400u)) - k1152;
            p[4 * m + 1] = as_h2(__builtin_amdgcn_perm(magic, hi, 0x04020400u)) * k16 - k18432;
            p[4 * m + 2] = as_h2(__builtin_amdgcn_perm(magic, lo, 0x04030401u)) - k1152;
            p[4 * m + 3] = as_h2(__builtin_amdgcn_perm(magic, hi, 0x04030401u)) * k16 - k18432;
        }
    }
}

// Six-bit scale (first) and min of Q4_K sub-block J from the packed bytes held
// as dwords s1 (bytes 0..3), s2 (4..7), s3 (8..11): J < 4 in the low six bits
// of bytes J and J + 4; J >= 4 a nibble of byte J + 4 under the top two bits
// of bytes J - 4 (scale) and J (min).
template <int J>
__device__ __forceinline__ void q4k_scale_min(uint32_t s1, uint32_t s2, uint32_t s3,
                                              uint32_t &sc, uint32_t &mn) {
    if constexpr (J < 4) {
        sc = __builtin_amdgcn_ubfe(s1, 8 * J, 6);
        mn = __builtin_amdgcn_ubfe(s2, 8 * J, 6);
    } else {
        constexpr int j = J - 4;
        sc = __builtin_amdgcn_ubfe(s3, 8 * j, 4) | __builtin_amdgcn_ubfe(s1, 8 * j + 6, 2) << 4;
        mn = __builtin_amdgcn_ubfe(s3, 8 * j + 4, 4) | __builtin_amdgcn_ubfe(s2, 8 * j + 6, 2) << 4;
    }
}

// The 16 pairs (pair order) of Q4_K sub-block 2c + H from the group's code
// dwords g[0..7], each pair = 1024 + q or, for pairs j = 1, 3, 1024 + 16 q
// (the caller subtracts 1024).  Elements 4m.. of the sub-block sit in dword m,
// elements 16 + 4m.. in dword 4 + m; low nibbles for H = 0, high for H = 1.
template <int H>
__device__ __forceinline__ void q4k_raw_pairs(const uint32_t *g, uint32_t *r, uint32_t magic) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t c0 = g[m], c1 = g[4 + m];
        if constexpr (H == 0) {
            r[4 * m + 0] = and_or(c0, 0x000F000Fu, magic);
            r[4 * m + 1] = and_or(c1 << 4, 0x00F000F0u, magic);
            r[4 * m + 2] = and_or(c0 >> 8, 0x000F000Fu, magic);
            r[4 * m + 3] = and_or(c1 >> 4, 0x00F000F0u, magic);
        } else {
            r[4 * m + 0] = and_or(c0 >> 4, 0x000F000Fu, magic);
            r[4 * m + 1] = and_or(c1, 0x00F000F0u, magic);
            r[4 * m + 2] = and_or(c0 >> 12, 0x000F000Fu, magic);
            r[4 * m + 3] = and_or(c1 >> 8, 0x00F000F0u, magic);
        }
    }
}

template <int Q, int B>
__device__ __forceinline__ float decode_pairs(const uint32_t *w, h2 *p, uint32_t magic) {
    uint32_t q[Q == FW_Q4_0 ? 4 : 8];
    const float d = block_codes<Q, B>(w, q);
    codes_to_pairs<Q>(q, p, magic);
    return d;
}

// The exponent bits decode_pairs ORs in: 0x6400 per half (fp16 1024), Q4_0 / Q4_K.
// For Q8_0 the same register serves as the 0x64 byte source of v_perm.
template <int Q> __device__ __forceinline__ uint32_t pair_magic() {
    return Q == FW_Q8_0 ? 0x64646464u : 0x64006400u;
}

// ---------------------------------------------------------------------------
// Launchers (defined in the .hip files).  All enqueue on `s` and return the
// launch's hipError_t.
hipError_t launch_logits(const fw_moe_desc &d, int T, const void *x, const void *wr,
                         const float *bias, float *logits, hipStream_t s);
hipError_t launch_topk(const fw_moe_desc &d, int T, const float *logits, int32_t *ids,
                       float *w, hipStream_t s);
// Pair counts above which the permutation runs as three multi-workgroup
// kernels (count, per-expert scan, scatter) instead of one workgroup.
constexpr int kPermChunk = 1024;
constexpr int kPermOneBlockMaxP = 2048;
inline int perm_blocks(long long P) { return (int)((P + kPermChunk - 1) / kPermChunk); }
hipError_t launch_permute(const fw_moe_desc &d, int T, const int32_t *ids, int32_t *offsets,
                          int32_t *sorted, int32_t *inv, WsHeader *hdr, int32_t *perm,
                          hipStream_t s);
hipError_t launch_clear_status(WsHeader *hdr, hipStream_t s);
hipError_t launch_copy_status(const WsHeader *hdr, int32_t *status, hipStream_t s);

struct FwdArgs {
    fw_moe_desc d;
    int T, P;
    int path;
    const void *x;
    const uint8_t *wg, *wu, *wd, *sg, *su, *sd;
    const float *topk_w;
    const int32_t *offsets, *sorted, *inv;
    float *out;
    char *ws;
    WsLayout L;
};
hipError_t launch_prepare(const FwdArgs &a, hipStream_t s);
// gate/up launchers: routed_done (may be null) is recorded between the
// routed experts' launch and the shared expert's
hipError_t launch_gemv_gate_up(const FwdArgs &a, hipEvent_t routed_done, hipStream_t s);
hipError_t launch_gemv_down(const FwdArgs &a, hipStream_t s);
hipError_t launch_gemm_gate_up(const FwdArgs &a, hipEvent_t routed_done, hipStream_t s);
hipError_t launch_gemm_down(const FwdArgs &a, hipStream_t s);
hipError_t launch_combine(const FwdArgs &a, hipStream_t s);
// MXFP8 expert activations (FW_ACT_MXFP8): the staging and the block-scaled
// grouped GEMMs (gemm_mx.hip); the launchers above hand over to these.
hipError_t launch_prepare_mx8(const FwdArgs &a, hipStream_t s);
hipError_t launch_gemm_mx_gate_up(const FwdArgs &a, hipEvent_t routed_done, hipStream_t s);
hipError_t launch_gemm_mx_down(const FwdArgs &a, hipStream_t s);
// int8 expert activations (FW_ACT_INT8): the staging and the int8-MFMA
// grouped GEMMs (gemm_i8.hip); the launchers above hand over to these.
hipError_t launch_prepare_i8(const FwdArgs &a, hipStream_t s);
hipError_t launch_gemm_i8_gate_up(const FwdArgs &a, hipEvent_t routed_done, hipStream_t s);
hipError_t launch_gemm_i8_down(const FwdArgs &a, hipStream_t s);
// fw_moe_layer's fused decode front end (top-k + permutation + staging in one
// launch): taken when the forward runs the GEMV family and the pairs fit the
// one-workgroup permutation.
bool decode_front_fits(const fw_moe_desc &d, int T, int path);
hipError_t launch_decode_front(const FwdArgs &a, const float *logits, int32_t *ids, float *w,
                               int32_t *offsets, int32_t *sorted, int32_t *inv, hipStream_t s);

}  // namespace fw
