// Forward, GEMV family (decode-sized batches): dequant-fused expert projections
// that read each active expert's blocks once.  Decode is bandwidth-bound (the
// pages' runtime counts its cost in weight bytes moved per token -- Flyweight
// 0.2.0 "Quantization"), so the kernels are built around HBM streaming:
//
//  - work items are (row chunk, 64-row weight tile) pairs: a row chunk is up to
//    two rows of one expert's segment of the sorted pair list (built on the
//    device), a weight tile 64 consecutive rows of that expert's matrix; the
//    grid is sized to the resident capacity and each workgroup walks the items
//    g, g + grid, ... so no workgroup pays a cold start twice;
//  - the S wavefronts of a workgroup split the reduction dimension: wavefront w
//    takes every S-th 256-element unit (8 GGUF blocks, 16-byte aligned), so the
//    wavefronts fetch adjacent units of the same rows together;
//  - weights move HBM -> LDS with global_load_lds_dwordx4 (each instruction
//    reads 1 KB of consecutive row bytes, so every cache line fetched is used
//    whole) through D buffers per wavefront; the batch stream runs across item
//    boundaries, so D batches stay in flight while one is consumed from
//    registers.  The LDS read of a batch waits only for that batch (vmcnt
//    counts the younger ones), written with the wait in the same asm block;
//  - lane r reads row r's unit from LDS (row strides of 144 / 272 bytes are
//    bank-conflict-free for 16 lanes); codes become exact fp16 pairs in
//    registers (decode_pairs) and meet the activation pairs in
//    v_dot2c_f32_f16 with fp32 accumulation; the fp16 block scale multiplies
//    each block's partial sum once;
//  - the activations of the chunk's rows are the same for every lane: they are
//    read with scalar loads and enter each dot as the scalar operand;
//  - partial sums of the S wavefronts meet in LDS and are added in wavefront
//    order, so results are deterministic.
// Gate and up rows of the same feature share a lane, so SiLU(g)*u is formed in
// registers (the fused gate/up pass that shares each activation load:
// Flyweight 0.2.0 "Current limitations").
#include <math.h>

#include <mutex>

#include "common.h"

namespace fw {
namespace {


typedef __attribute__((address_space(4))) const uint32_t cu32;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const uint4 *lds_cptr;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Stage unit u of the 64 rows starting at `tile` (row stride `rowbytes`) into
// buf[64 * X4] as [row][X4 x 16 bytes]: instruction i moves chunks
// c = 64 i + lane, chunk c being piece c % X4 of row c / X4.
template <int Q>
__device__ __forceinline__ void stage_unit(uint4 *buf, const uint8_t *tile, uint32_t rowbytes,
                                           int u, int lane, const uint8_t *stile = nullptr) {
    constexpr int X4 = QT<Q>::kUnitX4;
    if constexpr (Q == FW_MXFP4) {
        // pieces 0..7: the row's 128 code bytes of unit u; piece 8: the
        // 16-byte aligned piece holding its 8 scales (stile: the tile's first
        // scale row, 8-byte aligned; rows of rowbytes / 16 scale bytes)
#pragma unroll
        for (int i = 0; i < X4; ++i) {
            const uint32_t c = i * kWave + lane, row = c / X4, piece = c % X4;
            const uint8_t *src =
                piece < 8 ? tile + (row * rowbytes + (uint32_t)u * 128u + piece * 16)
                          : (const uint8_t *)((uintptr_t)(stile + row * (rowbytes / 16) + 8u * u) &
                                              ~(uintptr_t)15);
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + i * kWave), 16, 0, 0);
        }
        return;
    }
    if constexpr (Q == FW_Q6_K) {
        // 2-byte aligned units: row r's unit starts at byte o_r = mis + r *
        // rowbytes + 210 u of the 16-byte aligned base below the tile; its 14
        // covering pieces start at o_r & ~15.  The first and last piece each
        // hold a byte of the unit, so no 16-byte granule outside the unit's
        // own is touched.
        const uint8_t *base = (const uint8_t *)((uintptr_t)tile & ~(uintptr_t)15);
        const uint32_t mis = (uint32_t)(uintptr_t)tile & 15u;
#pragma unroll
        for (int i = 0; i < X4; ++i) {
            const uint32_t c = i * kWave + lane, row = c / X4, piece = c % X4;
            const uint32_t o = mis + row * rowbytes + (uint32_t)u * QT<Q>::kUnitBytes;
            __builtin_amdgcn_global_load_lds(base + ((o & ~15u) + piece * 16),
                                             (lds_void *)(buf + i * kWave), 16, 0, 0);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < X4; ++i) {
        // uniform base + 32-bit lane offset: the SGPR-base addressing form
        const uint32_t c = i * kWave + lane, row = c / X4, piece = c % X4;
        const uint32_t off = row * rowbytes + (uint32_t)u * QT<Q>::kUnitBytes + piece * 16;
        __builtin_amdgcn_global_load_lds(tile + off, (lds_void *)(buf + i * kWave), 16, 0, 0);
    }
}

// Row `lane`'s unit from a staged batch, once at most N vector loads of this
// wavefront are still outstanding (the batches staged after it).  The LDS
// reads and both waits sit in one asm block: the compiler cannot tell the LDS
// writes of global_load_lds apart and would otherwise wait for every batch.
// The block ends with lgkmcnt(0), so its outputs are complete when it ends and
// the buffer may be refilled right after.
template <int N>
__device__ __forceinline__ void wait_read_unit9(const uint4 *row, uint32_t *w) {
    const uint32_t a = (uint32_t)(uintptr_t)(lds_cptr)row;
    v4u r0, r1, r2, r3, r4, r5, r6, r7, r8;
    asm volatile(
        "s_waitcnt vmcnt(%9)\n\t"
        "ds_read_b128 %0, %10\n\t"
        "ds_read_b128 %1, %10 offset:16\n\t"
        "ds_read_b128 %2, %10 offset:32\n\t"
        "ds_read_b128 %3, %10 offset:48\n\t"
        "ds_read_b128 %4, %10 offset:64\n\t"
        "ds_read_b128 %5, %10 offset:80\n\t"
        "ds_read_b128 %6, %10 offset:96\n\t"
        "ds_read_b128 %7, %10 offset:112\n\t"
        "ds_read_b128 %8, %10 offset:128\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6),
          "=&v"(r7), "=&v"(r8)
        : "n"(N), "v"(a)
        : "memory");
    const v4u r[9] = {r0, r1, r2, r3, r4, r5, r6, r7, r8};
#pragma unroll
    for (int i = 0; i < 9; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[4 * i + j] = r[i][j];
}

template <int N>
__device__ __forceinline__ void wait_read_unit17(const uint4 *row, uint32_t *w) {
    const uint32_t a = (uint32_t)(uintptr_t)(lds_cptr)row;
    v4u r0, r1, r2, r3, r4, r5, r6, r7, r8, r9, r10, r11, r12, r13, r14, r15, r16;
    asm volatile(
        "s_waitcnt vmcnt(%17)\n\t"
        "ds_read_b128 %0, %18\n\t"
        "ds_read_b128 %1, %18 offset:16\n\t"
        "ds_read_b128 %2, %18 offset:32\n\t"
        "ds_read_b128 %3, %18 offset:48\n\t"
        "ds_read_b128 %4, %18 offset:64\n\t"
        "ds_read_b128 %5, %18 offset:80\n\t"
        "ds_read_b128 %6, %18 offset:96\n\t"
        "ds_read_b128 %7, %18 offset:112\n\t"
        "ds_read_b128 %8, %18 offset:128\n\t"
        "ds_read_b128 %9, %18 offset:144\n\t"
        "ds_read_b128 %10, %18 offset:160\n\t"
        "ds_read_b128 %11, %18 offset:176\n\t"
        "ds_read_b128 %12, %18 offset:192\n\t"
        "ds_read_b128 %13, %18 offset:208\n\t"
        "ds_read_b128 %14, %18 offset:224\n\t"
        "ds_read_b128 %15, %18 offset:240\n\t"
        "ds_read_b128 %16, %18 offset:256\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6),
          "=&v"(r7), "=&v"(r8), "=&v"(r9), "=&v"(r10), "=&v"(r11), "=&v"(r12), "=&v"(r13),
          "=&v"(r14), "=&v"(r15), "=&v"(r16)
        : "n"(N), "v"(a)
        : "memory");
    const v4u r[17] = {r0, r1, r2, r3, r4, r5, r6, r7, r8, r9, r10, r11, r12, r13, r14, r15, r16};
#pragma unroll
    for (int i = 0; i < 17; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) w[4 * i + j] = r[i][j];
}

// Activation pairs of block B of unit u for NTK token rows: one scalar load
// of 16 dwords per row.
template <int NTK>
__device__ __forceinline__ void load_x(uint32_t (*x)[16], cu32 *const *in, int u, int B) {
#pragma unroll
    for (int n = 0; n < NTK; ++n) {
        cu32 *xp = in[n] + (u * kUnit + 32 * B) / 2;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[n][i] = xp[i];
    }
}

template <int Q, int NTK, int B>
__device__ __forceinline__ void dot_block(const uint32_t *w, const uint32_t (*x)[16],
                                          uint32_t magic, float *acc) {
    h2 p[16];
    const float d = decode_pairs<Q, B>(w, p, magic);
#pragma unroll
    for (int n = 0; n < NTK; ++n) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s = __builtin_amdgcn_fdot2(p[i], as_h2(x[n][i]), s, false);
        acc[n] = fmaf(d, s, acc[n]);
    }
}

// Activation sets a unit's dot keeps in SGPRs: one row prefetches three blocks
// ahead (hiding a scalar-cache miss on long rows), two rows one block ahead
// (16 SGPRs per row and block, plus the block sum for Q4_K).
template <int NTK> constexpr int x_sets() { return NTK == 1 ? 4 : 2; }

// Q4_K unit (one super-block): sub-block J is block J of the unit in pair
// order.  Its exact code pairs meet the activation pairs in fp32 dot products,
// and the sub-block's scale and min apply once, in fp32:
//   acc += d * scale_J * sum(q x) - dmin * min_J * sum(x),
// sum(x) being the activation row's precomputed 32-element block sums (sum[n]:
// one fp32 per block, written by the kernel that produced the row).
template <int NTK>
__device__ __forceinline__ void dot_unit_q4k(const uint32_t *w, int u, cu32 *const *in,
                                             cu32 *const *sum, float *acc) {
    const uint32_t magic = pair_magic<FW_Q4_K>();
    const float d = half_bits_to_float(w[0] & 0xFFFFu), dmin = half_bits_to_float(w[0] >> 16);
    const h2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
    // activation pairs of a sub-block plus the block's sum, NB - 1 blocks ahead
    constexpr int NB = x_sets<NTK>();
    uint32_t xs[NB][NTK][17];
    auto load_xk = [&](uint32_t (*x)[17], int B) {
#pragma unroll
        for (int n = 0; n < NTK; ++n) {
            cu32 *xp = in[n] + (u * kUnit + 32 * B) / 2;
#pragma unroll
            for (int i = 0; i < 16; ++i) x[n][i] = xp[i];
            x[n][16] = sum[n][8 * u + B];
        }
    };
#pragma unroll
    for (int j = 0; j < NB - 1; ++j) load_xk(xs[j], j);
#define FW_SUB(J)                                                                    \
    {                                                                                \
        if (J + NB - 1 < 8) load_xk(xs[(J + NB - 1) % NB], J + NB - 1);              \
        const uint32_t(*CUR)[17] = xs[J % NB];                                       \
        uint32_t r[16], sc, mn;                                                      \
        q4k_raw_pairs<J % 2>(w + 4 + 8 * (J / 2), r, magic);                         \
        q4k_scale_min<J>(w[1], w[2], w[3], sc, mn);                                  \
        const float ds = d * (float)sc, dm = dmin * (float)mn;                       \
        _Pragma("unroll") for (int n = 0; n < NTK; ++n) {                            \
            float s = 0.f;                                                           \
            _Pragma("unroll") for (int i = 0; i < 16; ++i)                           \
                s = __builtin_amdgcn_fdot2(as_h2(r[i]) - k1024, as_h2(CUR[n][i]), s, \
                                           false);                                   \
            acc[n] = fmaf(ds, s, acc[n]);                                            \
            acc[n] = fmaf(-dm, __uint_as_float(CUR[n][16]), acc[n]);                 \
        }                                                                            \
    }                                                                                \
    __builtin_amdgcn_sched_barrier(0);
    FW_SUB(0)
    FW_SUB(1)
    FW_SUB(2)
    FW_SUB(3)
    FW_SUB(4)
    FW_SUB(5)
    FW_SUB(6)
    FW_SUB(7)
#undef FW_SUB
}

// acc[n] += (row's unit u) . (activation row n's unit u), n < NTK.  The
// activations of block B + NB - 1 are loaded while block B is consumed;
// scheduling barriers keep one block's pairs live at a time.
template <int Q, int NTK>
__device__ __forceinline__ void dot_unit_blocks(const uint32_t *w, int u, cu32 *const *in,
                                                float *acc) {
    const uint32_t magic = pair_magic<Q>();
    constexpr int NB = x_sets<NTK>();
    uint32_t xs[NB][NTK][16];
#pragma unroll
    for (int j = 0; j < NB - 1; ++j) load_x<NTK>(xs[j], in, u, j);
#define FW_BLOCK(B)                                                        \
    if (B + NB - 1 < 8) load_x<NTK>(xs[(B + NB - 1) % NB], in, u, B + NB - 1); \
    dot_block<Q, NTK, B>(w, xs[B % NB], magic, acc);                       \
    __builtin_amdgcn_sched_barrier(0);
    FW_BLOCK(0)
    FW_BLOCK(1)
    FW_BLOCK(2)
    FW_BLOCK(3)
    FW_BLOCK(4)
    FW_BLOCK(5)
    FW_BLOCK(6)
    FW_BLOCK(7)
#undef FW_BLOCK
}

// Row `lane`'s Q6_K unit from its staged pieces (the only batch in flight:
// Q6_K runs one buffer per wavefront), realigned so that w[i] holds bytes
// 4i .. 4i + 3 of the unit (i < 53).  sub: the unit's byte offset in the
// first piece (even, 0 .. 14).  The reads start at the dword holding the
// unit's first byte (a per-lane LDS address); a 2-byte offset is taken out
// with v_alignbyte.
__device__ __forceinline__ void read_unit_q6k(const uint4 *slot, uint32_t sub, uint32_t *w) {
    __builtin_amdgcn_s_waitcnt(7 << 4);   // vmcnt(0): the batch has landed
    const uint32_t *p = (const uint32_t *)((const uint8_t *)slot + (sub & 12u));
    uint32_t r[54];
#pragma unroll
    for (int i = 0; i < 54; ++i) r[i] = p[i];
    // every LDS read has returned before the buffer's next DMA is issued
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    const uint32_t sh = sub & 3u;
#pragma unroll
    for (int i = 0; i < 53; ++i) w[i] = __builtin_amdgcn_alignbyte(r[i + 1], r[i], sh);
}

// Q6_K unit (one super-block) in pair order: block B = 4h + k of the unit
// (half h, k = 0..3) takes its codes' low four bits from ql dwords
// 16h + 8 (k % 2) + m (elements 4m ..) and + 4 (elements 16 + 4m ..), nibble
// k / 2, and their top two bits from qh dwords 32 + 8h + m (+ 4), bits 2k.
// Four six-bit codes form in the bytes of one dword; two of them at a time
// become the exact fp16 pair 1024 + q (pairs j = 0, 2) or 1024 + 16 q (pairs
// j = 1, 3, whose activations carry 1/16).  Elements l < 16 of a block
// (pairs j = 0, 2) are sub-block 2B, the others 2B + 1: two dot sums per
// block, each scaled once by d * scale in fp32.
template <int NTK>
__device__ __forceinline__ void dot_unit_q6k(const uint32_t *w, int u, cu32 *const *in,
                                             float *acc) {
    const uint32_t magic = pair_magic<FW_Q6_K>();
    const float d = half_bits_to_float(w[52] & 0xFFFFu);
    const h2 k1056 = {(_Float16)1056.0f, (_Float16)1056.0f};
    const h2 k1536 = {(_Float16)1536.0f, (_Float16)1536.0f};
    constexpr int NB = x_sets<NTK>();
    uint32_t xs[NB][NTK][16];
#pragma unroll
    for (int j = 0; j < NB - 1; ++j) load_x<NTK>(xs[j], in, u, j);
#define FW_Q6B(B)                                                                        \
    {                                                                                    \
        if (B + NB - 1 < 8) load_x<NTK>(xs[(B + NB - 1) % NB], in, u, B + NB - 1);       \
        const uint32_t(*X)[16] = xs[B % NB];                                             \
        constexpr int H = (B) / 4, KK = (B) % 4;                                         \
        const uint32_t *ql = w + 16 * H + 8 * (KK % 2), *qh = w + 32 + 8 * H;            \
        h2 p[16];                                                                        \
        _Pragma("unroll") for (int m = 0; m < 4; ++m) {                                  \
            const uint32_t cl = and_or(ql[m] >> (4 * (KK / 2)), 0x0F0F0F0Fu,             \
                                       ((qh[m] >> (2 * KK)) & 0x03030303u) << 4);        \
            const uint32_t ch = and_or(ql[m + 4] >> (4 * (KK / 2)), 0x0F0F0F0Fu,         \
                                       ((qh[m + 4] >> (2 * KK)) & 0x03030303u) << 4);    \
            p[4 * m + 0] = as_h2(and_or(cl, 0x003F003Fu, magic)) - k1056;                \
            p[4 * m + 1] = as_h2(and_or(ch << 4, 0x03F003F0u, magic)) - k1536;           \
            p[4 * m + 2] = as_h2(and_or(cl >> 8, 0x003F003Fu, magic)) - k1056;           \
            p[4 * m + 3] = as_h2(and_or(ch >> 4, 0x03F003F0u, magic)) - k1536;           \
        }                                                                                \
        const float s0 = d * (float)(int)__builtin_amdgcn_sbfe(w[48 + (B) / 2], 16 * ((B) & 1), 8); \
        const float s1 = d * (float)(int)__builtin_amdgcn_sbfe(w[48 + (B) / 2], 16 * ((B) & 1) + 8, 8); \
        _Pragma("unroll") for (int n = 0; n < NTK; ++n) {                                \
            float lo = 0.f, hi = 0.f;                                                    \
            _Pragma("unroll") for (int m = 0; m < 4; ++m) {                              \
                lo = __builtin_amdgcn_fdot2(p[4 * m + 0], as_h2(X[n][4 * m + 0]), lo, false); \
                lo = __builtin_amdgcn_fdot2(p[4 * m + 2], as_h2(X[n][4 * m + 2]), lo, false); \
                hi = __builtin_amdgcn_fdot2(p[4 * m + 1], as_h2(X[n][4 * m + 1]), hi, false); \
                hi = __builtin_amdgcn_fdot2(p[4 * m + 3], as_h2(X[n][4 * m + 3]), hi, false); \
            }                                                                            \
            acc[n] = fmaf(s0, lo, acc[n]);                                               \
            acc[n] = fmaf(s1, hi, acc[n]);                                               \
        }                                                                                \
    }                                                                                    \
    __builtin_amdgcn_sched_barrier(0);
    FW_Q6B(0)
    FW_Q6B(1)
    FW_Q6B(2)
    FW_Q6B(3)
    FW_Q6B(4)
    FW_Q6B(5)
    FW_Q6B(6)
    FW_Q6B(7)
#undef FW_Q6B
}

// MXFP4 unit: w[0..31] the 128 code bytes (block B in w[4B .. 4B + 3],
// element j of a block in nibble j % 2 of byte j / 2), the unit's 8 scales
// in w[so], w[so + 1].  Pair 4m + j takes bytes 2m, 2m + 1 of the block's
// first (j = 0, 2) or second (j = 1, 3) 16 bytes, low nibbles for j < 2.  A
// nibble becomes the fp16 whose bits 11..9 are the code's magnitude bits and
// bit 15 its sign: exactly E2M1(code) * 2^-14 (the two smallest magnitudes
// land on fp16 subnormals, 0 and 2^-15).  The exact products meet the
// activations in fp32 dot sums, and the block's 2^(scale - 127) (x 2^14, and
// x 16 for pairs j = 1, 3) applies once, exactly, by ldexp.
__device__ __forceinline__ uint32_t e2m1_pair_lo(uint32_t g) {   // nibbles at bits 0, 16
    return and_or(g << 9, 0x0E000E00u, (g << 12) & 0x80008000u);
}
__device__ __forceinline__ uint32_t e2m1_pair_hi(uint32_t g) {   // nibbles at bits 4, 20
    return and_or(g << 5, 0x0E000E00u, (g << 8) & 0x80008000u);
}

template <int NTK>
__device__ __forceinline__ void dot_unit_mxfp4(const uint32_t *w, int u, cu32 *const *in,
                                               float *acc, int so) {
    const uint32_t sc0 = so ? w[34] : w[32], sc1 = so ? w[35] : w[33];
    constexpr int NB = x_sets<NTK>();
    uint32_t xs[NB][NTK][16];
#pragma unroll
    for (int j = 0; j < NB - 1; ++j) load_x<NTK>(xs[j], in, u, j);
#define FW_MXB(B)                                                                        \
    {                                                                                    \
        if (B + NB - 1 < 8) load_x<NTK>(xs[(B + NB - 1) % NB], in, u, B + NB - 1);       \
        const uint32_t(*X)[16] = xs[B % NB];                                             \
        h2 p[16];                                                                        \
        _Pragma("unroll") for (int m = 0; m < 4; ++m) {                                  \
            /* bytes 2m, 2m + 1 of the block's halves moved to bytes 0 and 2 */          \
            const uint32_t sel = (m & 1) ? 0x0C030C02u : 0x0C010C00u;                    \
            const uint32_t g0 = __builtin_amdgcn_perm(0u, w[4 * (B) + m / 2], sel);      \
            const uint32_t g1 = __builtin_amdgcn_perm(0u, w[4 * (B) + 2 + m / 2], sel);  \
            p[4 * m + 0] = as_h2(e2m1_pair_lo(g0));                                      \
            p[4 * m + 1] = as_h2(e2m1_pair_lo(g1));                                      \
            p[4 * m + 2] = as_h2(e2m1_pair_hi(g0));                                      \
            p[4 * m + 3] = as_h2(e2m1_pair_hi(g1));                                      \
        }                                                                                \
        const int ex = (int)__builtin_amdgcn_ubfe((B) < 4 ? sc0 : sc1, 8 * ((B) & 3), 8) - 113; \
        _Pragma("unroll") for (int n = 0; n < NTK; ++n) {                                \
            float lo = 0.f, hi = 0.f;                                                    \
            _Pragma("unroll") for (int m = 0; m < 4; ++m) {                              \
                lo = __builtin_amdgcn_fdot2(p[4 * m + 0], as_h2(X[n][4 * m + 0]), lo, false); \
                lo = __builtin_amdgcn_fdot2(p[4 * m + 2], as_h2(X[n][4 * m + 2]), lo, false); \
                hi = __builtin_amdgcn_fdot2(p[4 * m + 1], as_h2(X[n][4 * m + 1]), hi, false); \
                hi = __builtin_amdgcn_fdot2(p[4 * m + 3], as_h2(X[n][4 * m + 3]), hi, false); \
            }                                                                            \
            acc[n] += __builtin_amdgcn_ldexpf(lo, ex) + __builtin_amdgcn_ldexpf(hi, ex + 4); \
        }                                                                                \
    }                                                                                    \
    __builtin_amdgcn_sched_barrier(0);
    FW_MXB(0)
    FW_MXB(1)
    FW_MXB(2)
    FW_MXB(3)
    FW_MXB(4)
    FW_MXB(5)
    FW_MXB(6)
    FW_MXB(7)
#undef FW_MXB
}

template <int Q, int NTK>
__device__ __forceinline__ void dot_unit(const uint32_t *w, int u, cu32 *const *in,
                                         cu32 *const *sum, float *acc) {
    if constexpr (Q == FW_Q4_K)
        dot_unit_q4k<NTK>(w, u, in, sum, acc);
    else if constexpr (Q == FW_Q6_K)
        dot_unit_q6k<NTK>(w, u, in, acc);
    else
        dot_unit_blocks<Q, NTK>(w, u, in, acc);
}

// What a wavefront needs of one work item: the 64-row weight tile of each
// matrix, the activation rows of the item's chunk, and where outputs go.
struct Item {
    const uint8_t *ta, *tb;
    cu32 *in[kGemvTokens];
    cu32 *sum[kGemvTokens];   // Q4_K: the rows' 32-element block sums
    int ex[kGemvTokens];      // power-of-two exponent each input row is scaled by
    int rb, nt, tile;
    bool bad;
};

// The weight tiles (one per matrix) of work item `item`.
__device__ __forceinline__ void tile_bases(int item, const uint8_t *wa, const uint8_t *wb,
                                           const int4 *tiles, size_t rowbytes, size_t esz,
                                           int tpg, int shared, const uint8_t *&ta,
                                           const uint8_t *&tb) {
    const int chunk = item / tpg;
    size_t off = (size_t)(item % tpg) * kWave * rowbytes;
    if (!shared) off += (size_t)ld_const(&tiles[chunk].x) * esz;
    ta = wa + off;
    tb = wb + off;
}

template <bool GU>
__device__ __forceinline__ Item get_item(int item, const uint8_t *wa, const uint8_t *wb,
                                         const int4 *tiles, const int32_t *sorted,
                                         const _Float16 *xin, const float *isum,
                                         const int32_t *iexp, size_t rowbytes, size_t esz,
                                         int tpg, int K, int k, int P, int shared,
                                         int shared_rows) {
    Item it;
    const int chunk = item / tpg;
    it.tile = item % tpg;
    size_t off = (size_t)it.tile * kWave * rowbytes;
    if (shared) {
        it.rb = chunk * kGemvTokens;
        it.nt = min(kGemvTokens, shared_rows - it.rb);
    } else {
        const int4 c = ld_const(tiles + chunk);   // (expert, first row, rows)
        off += (size_t)c.x * esz;
        it.rb = c.y;
        it.nt = c.z;
    }
    it.ta = wa + off;
    it.tb = wb + off;
    it.bad = false;
#pragma unroll
    for (int n = 0; n < kGemvTokens; ++n) {
        const int r = it.rb + min(n, it.nt - 1);
        int t = r;   // the down projection reads row r of its input
        if (GU && !shared) {
            const int q = ld_const(sorted + r);
            it.bad |= (unsigned)q >= (unsigned)P;
            t = (unsigned)q < (unsigned)P ? q / k : 0;
        }
        it.in[n] = (cu32 *)(xin + (size_t)t * K);
        it.sum[n] = (cu32 *)(isum + (size_t)t * (K / 32));
        it.ex[n] = ld_const(iexp + t);
    }
    return it;
}

// LDS read of a staged batch with at most `ahead` younger batches (LOADS
// vector loads each) still in flight; D - 1 >= ahead.
template <int Q, int D>
__device__ __forceinline__ void wait_read(const uint4 *row, int ahead, uint32_t *w) {
    constexpr int X4 = QT<Q>::kUnitX4;
    static_assert(X4 * (D - 1) <= 63, "vmcnt holds at most 63");
#define FW_WAIT(A)                                                                 \
    if (D > A && ahead >= A) {                                                    \
        if constexpr (X4 == 9) wait_read_unit9<(D > A ? A * X4 : 0)>(row, w);     \
        else wait_read_unit17<(D > A ? A * X4 : 0)>(row, w);                      \
        return;                                                                   \
    }
    FW_WAIT(3)
    FW_WAIT(2)
    FW_WAIT(1)
#undef FW_WAIT
    if constexpr (X4 == 9) wait_read_unit9<0>(row, w);
    else wait_read_unit17<0>(row, w);
}

// Work items are (row chunk, 64-row weight tile) pairs, item = chunk * tpg +
// tile; a chunk is up to kGemvTokens rows of one expert's segment of the
// sorted pair list (routed) or of the token rows (shared expert).  Workgroup
// g takes items g, g + grid, ...; its S wavefronts split each item's units,
// and each streams its batches (NV matrices per unit) through D LDS buffers
// with the stream running across item boundaries.
template <int Q, bool GU, int S, int D>
__global__ __launch_bounds__(kWave *S) void gemv_kernel(
    const uint8_t *__restrict__ wa, const uint8_t *__restrict__ wb,
    const int4 *__restrict__ tiles, WsHeader *__restrict__ hdr,
    const int32_t *__restrict__ sorted, const _Float16 *__restrict__ xin,
    _Float16 *__restrict__ hout, float *__restrict__ yout, int K, int N, int k, int P,
    int tpg, int max_chunks, int shared, int shared_rows, int ks, int *__restrict__ split_cnt,
    float *__restrict__ split_part, const float *__restrict__ isum, float *__restrict__ osum,
    const int32_t *__restrict__ iexp, int32_t *__restrict__ oexp, size_t sreg) {
    constexpr int X4 = QT<Q>::kUnitX4;
    constexpr int NV = GU ? 2 : 1;
    constexpr int NT = kGemvTokens;
    __shared__ uint4 stage[S][D][kWave * X4];
    __shared__ float red[S > 1 ? S - 1 : 1][NV * NT][kWave];
    const int wave = wave_id(), lane = threadIdx.x % kWave;
    const size_t rowbytes = QT<Q>::row_bytes(K);
    const size_t esz = (size_t)N * rowbytes;
    const uint8_t *wbb = GU ? wb : wa;
    // the device-written chunk count is clamped to the bound the launch (its
    // split-K slices and their counters and partials) was sized for: corrupt
    // expert_offsets can make the schedule claim more
    const int n_chunks = shared ? (shared_rows + NT - 1) / NT
                                : min(ld_const(&hdr->n_tiles), max_chunks);
    const int n_items = n_chunks * tpg * ks;
    const int g0 = blockIdx.x, G = gridDim.x;
    if (g0 >= n_items) return;
    const int my_items = (n_items - g0 + G - 1) / G;
    const int us = (K / kUnit) / ks;        // units per reduction slice
    const int nb = NV * (us / S);           // batches per wavefront per item
    const int total = my_items * nb;
    const uint32_t rb32 = (uint32_t)rowbytes;
    // MXFP4: a tile's first scale row, from its first code row (row bytes K/2
    // of codes, K/32 of scales; the scales of a matrix start sreg bytes in)
    auto scale_tile = [&](const uint8_t *mat, const uint8_t *tile) {
        return Q == FW_MXFP4 ? mat + sreg + (size_t)(tile - mat) / 16 : nullptr;
    };
    // staging cursor: batch js overall, bs within its item (D ahead of use);
    // only the item's two weight tiles are needed to stage
    int js = 0, is_ = 0, bs = 0;
    const uint8_t *sa, *sb;
    tile_bases(g0 / ks, wa, wbb, tiles, rowbytes, esz, tpg, shared, sa, sb);
#define FW_STAGE_NEXT()                                                                     \
    do {                                                                                    \
        if (bs == nb) {                                                                     \
            bs = 0;                                                                         \
            ++is_;                                                                          \
            tile_bases((g0 + is_ * G) / ks, wa, wbb, tiles, rowbytes, esz, tpg, shared, sa, sb); \
        }                                                                                   \
        stage_unit<Q>(stage[wave][js % D], (NV == 2 && (bs & 1)) ? sb : sa, rb32,           \
                      ((g0 + is_ * G) % ks) * us + wave + (bs / NV) * S, lane,              \
                      (NV == 2 && (bs & 1)) ? scale_tile(wbb, sb) : scale_tile(wa, sa));    \
        ++bs;                                                                               \
        ++js;                                                                               \
    } while (0)
    for (int j = 0; j < D && j < total; ++j) FW_STAGE_NEXT();

    int j = 0;
    for (int i = 0; i < my_items; ++i) {
        const int item = g0 + i * G, ct = item / ks, slice = item % ks;
        const Item it = get_item<GU>(ct, wa, wbb, tiles, sorted, xin, isum, iexp, rowbytes, esz,
                                     tpg, K, k, P, shared, shared_rows);
        if (it.bad && threadIdx.x == 0) atomicOr(&hdr->status, FW_STATUS_BAD_PAIR);
        float acc[NV][NT];
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[v][n] = 0.f;
        for (int b = 0; b < nb; ++b, ++j) {
            uint32_t w[4 * X4];
            const int u = slice * us + wave + (b / NV) * S;
            int so = 0;   // MXFP4: the dword of the scale piece holding the unit's scales
            if constexpr (Q == FW_MXFP4) {
                const uint8_t *st = (NV == 2 && (b & 1)) ? scale_tile(wbb, it.tb)
                                                         : scale_tile(wa, it.ta);
                so = (int)(((uintptr_t)st + (uint32_t)lane * (rb32 / 16) + 8u * (uint32_t)u) >> 2) & 2;
            }
            if constexpr (Q == FW_Q6_K) {
                const uint8_t *tl = (NV == 2 && (b & 1)) ? it.tb : it.ta;
                const uint32_t sub =
                    ((uint32_t)(uintptr_t)tl + (uint32_t)lane * rb32 + 210u * (uint32_t)u) & 15u;
                read_unit_q6k(&stage[wave][j % D][lane * X4], sub, w);
            } else {
                wait_read<Q, D>(&stage[wave][j % D][lane * X4], min(D - 1, total - 1 - j), w);
            }
            if (js < total) FW_STAGE_NEXT();
            float *a = acc[NV == 2 ? (b & 1) : 0];
            if constexpr (Q == FW_MXFP4) {
                if (it.nt == 1) dot_unit_mxfp4<1>(w, u, it.in, a, so);
                else dot_unit_mxfp4<2>(w, u, it.in, a, so);
            } else {
                if (it.nt == 1) dot_unit<Q, 1>(w, u, it.in, it.sum, a);
                else dot_unit<Q, 2>(w, u, it.in, it.sum, a);
            }
        }
        // partial sums of waves 1..S-1 meet wave 0's in LDS, added in wave order
        if (S > 1) {
            if (wave > 0) {
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int n = 0; n < NT; ++n) red[wave - 1][v * NT + n][lane] = acc[v][n];
            }
            __syncthreads();
            if (wave == 0) {
#pragma unroll
                for (int s = 0; s < S - 1; ++s)
#pragma unroll
                    for (int v = 0; v < NV; ++v)
#pragma unroll
                        for (int n = 0; n < NT; ++n) acc[v][n] += red[s][v * NT + n][lane];
            }
        }
        // split-K: every slice leaves its sums in split_part; the last slice
        // of the tile to arrive (an integer counter) adds all slices in slice
        // order and writes the outputs
        bool out = wave == 0;
        if (ks > 1 && wave == 0) {
            float *part = split_part + (size_t)ct * ks * (NV * NT * kWave);
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    part[((size_t)slice * NV * NT + v * NT + n) * kWave + lane] = acc[v][n];
            __threadfence();
            int old = 0;
            if (lane == 0) old = atomicAdd(&split_cnt[ct], 1);
            old = __builtin_amdgcn_readfirstlane(old);
            out = old == ks - 1;
            if (out) {
                __threadfence();
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[v][n] = 0.f;
                for (int sl = 0; sl < ks; ++sl)
#pragma unroll
                    for (int v = 0; v < NV; ++v)
#pragma unroll
                        for (int n = 0; n < NT; ++n)
                            acc[v][n] += part[((size_t)sl * NV * NT + v * NT + n) * kWave + lane];
                if (lane == 0) split_cnt[ct] = 0;   // ready for the next launch
            }
        }
        if (out) {
            const int row = it.tile * kWave + lane;
            bool range = false;
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if (n < it.nt) {
                    const size_t r = (size_t)(it.rb + n);
                    const int e = it.ex[n];
                    if constexpr (GU) {
                        // g and u at the token's own scale (exact), SwiGLU in
                        // fp32, h stored at 2^(2e) (pairs j = 1, 3 at 1/16)
                        const float gv = __builtin_amdgcn_ldexpf(acc[0][n], -e);
                        const float up = __builtin_amdgcn_ldexpf(acc[NV - 1][n], -e);
                        const float a = gv / (1.0f + __expf(-gv)) * up;
                        const _Float16 ah =
                            (_Float16)__builtin_amdgcn_ldexpf(a, 2 * e - ((row & 16) ? 4 : 0));
                        range |= (__builtin_bit_cast(uint16_t, ah) & 0x7C00u) == 0x7C00u;
                        hout[r * N + (row & ~31) + pair_pos(row & 31)] = ah;
                        if (it.tile == 0 && lane == 0) oexp[r] = 2 * e;
                        if (osum) {
                            // 32-element block sums of the stored values (a Q4_K
                            // down projection's min term), in a fixed order
                            float v = (row & 16) ? 16.0f * (float)ah : (float)ah;
#pragma unroll
                            for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o);
                            if ((lane & 31) == 0) osum[r * (N / 32) + row / 32] = v;
                        }
                    } else {
                        yout[r * N + row] = __builtin_amdgcn_ldexpf(acc[0][n], -e);
                    }
                }
            }
            if (GU && range) atomicOr(&hdr->status, FW_STATUS_RANGE);
        }
        if (S > 1) __syncthreads();   // red[] is reused by the next item
    }
#undef FW_STAGE_NEXT
}

// Wavefronts per workgroup: the reduction dimension is split into S ranges of
// whole 256-element units.
int pick_split(int units) {
    for (int s : {4, 3, 2})
        if (units % s == 0) return s;
    return 1;
}

// Properties of the current device, queried once per device (thread-safe)
// and read-only after that.
int cu_count() {
    static std::once_flag once[kMaxDevices];
    static int cus[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    std::call_once(once[dev], [dev] {
        int n = 0;
        cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                               hipSuccess && n > 0 ? n : 256;
    });
    return cus[dev];
}

// Resident workgroups per CU of one kernel, per device (registers and LDS).
template <typename K>
int resident_per_cu(K kernel, int threads) {
    static std::once_flag once[kMaxDevices];
    static int res[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1;
    std::call_once(once[dev], [&] {
        int n = 0;
        res[dev] = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) ==
                               hipSuccess && n > 0 ? n : 1;
    });
    return res[dev];
}

// isum: the input rows' 32-element block sums (Q4_K weights), osum: where
// the gate/up pass leaves those of its output rows (a Q4_K down projection);
// either may be null.
template <int Q, bool GU, int S, int D>
void launch_sd(const FwdArgs &a, const uint8_t *wa, const uint8_t *wb, const _Float16 *xin,
               _Float16 *hout, float *yout, int K, int N, int max_chunks, int per_cu, int ks,
               int shared, const float *isum, float *osum, const int32_t *iexp, int32_t *oexp,
               hipStream_t s) {
    const int tpg = N / kWave;
    const long long items = (long long)max_chunks * tpg;
    // workgroups per CU: what the LDS pipeline asks for, but no more than
    // registers and LDS let be resident at once (the schedule is persistent)
    per_cu = std::min(per_cu, resident_per_cu(gemv_kernel<Q, GU, S, D>, kWave * S));
    const long long work = items * ks, slots = (long long)per_cu * cu_count();
    // gate/up: equal rounds, every workgroup takes the same number of items,
    // so no last partial round of items runs latency-bound after the rest
    // (decode T=16: about 1100 items on 1024 slots, 40.7 -> 39.4 us); the
    // down projection keeps every slot busy (equal rounds there leave fewer
    // workgroups resident: 25.4 -> 28.0 us)
    const long long rounds = (work + slots - 1) / slots;
    const int grid = (int)std::max(1LL, GU ? (work + rounds - 1) / rounds : std::min(work, slots));
    gemv_kernel<Q, GU, S, D><<<grid, kWave * S, 0, s>>>(
        wa, wb, (const int4 *)(a.ws + a.L.tiles), (WsHeader *)a.ws, a.sorted, xin, hout, yout,
        K, N, a.d.top_k, a.P, tpg, max_chunks, shared, shared ? a.T : 0, ks,
        (int *)(a.ws + a.L.split_cnt),
        (float *)(a.ws + a.L.split_part), isum, osum, iexp, oexp,
        (size_t)(shared ? 1 : a.d.n_experts) * N * (size_t)(K / 2));
}

// LDS is the in-flight buffer: about 144 KB of DMA batches per CU keeps HBM
// busy.  Few items per CU (small batches, few active experts) get deep
// per-wavefront pipelines; many items get more resident workgroups instead.
template <int Q, bool GU, int S>
void launch_s(const FwdArgs &a, const uint8_t *wa, const uint8_t *wb, const _Float16 *xin,
              _Float16 *hout, float *yout, int K, int N, int max_chunks, int shared,
              const float *isum, float *osum, const int32_t *iexp, int32_t *oexp,
              hipStream_t s) {
    constexpr int X4 = QT<Q>::kUnitX4;
    const long long items = (long long)max_chunks * (N / kWave);
    // far too few items to occupy the CUs (the shared expert of a one-token
    // batch): split the reduction dimension into slices of whole units (each
    // wavefront keeps at least one unit per slice).  The slices meet through
    // memory with device-scope fences, which costs more than it gains once
    // there are a few items per CU.
    int ks = 1;
    if (items <= kSplitTiles && items * 4 < cu_count()) {
        const int per_wave = (K / kUnit) / S;
        for (int c = kSplitSlicesMax; c > 1; --c)
            if (per_wave % c == 0 && items * (c - 1) < 2LL * cu_count()) {
                ks = c;
                break;
            }
    }
    const double per_cu = (double)items * ks / cu_count();
    // workgroups per CU that the kernel's static LDS allows
    const size_t batch = (size_t)S * kWave * X4 * 16;   // one batch of every wavefront
    const size_t red = (size_t)std::max(S - 1, 1) * (GU ? 2 : 1) * kGemvTokens * kWave * 4;
    auto fit = [&](int d) { return (int)std::max<size_t>(1, (160 * 1024) / (batch * d + red)); };
    // 9 KB batches (Q4_0, Q4_K): depth 2 between 1.5 and 3 items per CU, else
    // 1 (deeper pipelines for one-token batches measured slower once the
    // one-row dots prefetch their activations further ahead); 17 KB batches
    // (Q8_0): depth 1
    if (X4 == 9 && per_cu >= 1.5 && per_cu < 3.0)
        launch_sd<Q, GU, S, 2>(a, wa, wb, xin, hout, yout, K, N, max_chunks, fit(2), ks, shared, isum, osum, iexp, oexp, s);
    else
        launch_sd<Q, GU, S, 1>(a, wa, wb, xin, hout, yout, K, N, max_chunks, fit(1), ks, shared, isum, osum, iexp, oexp, s);
}

template <int Q, bool GU>
void launch(const FwdArgs &a, const uint8_t *wa, const uint8_t *wb, const _Float16 *xin,
            _Float16 *hout, float *yout, int K, int N, int max_chunks, int shared,
            const float *isum, float *osum, const int32_t *iexp, int32_t *oexp, hipStream_t s) {
    switch (pick_split(K / kUnit)) {
        case 4: launch_s<Q, GU, 4>(a, wa, wb, xin, hout, yout, K, N, max_chunks, shared, isum, osum, iexp, oexp, s); break;
        case 3: launch_s<Q, GU, 3>(a, wa, wb, xin, hout, yout, K, N, max_chunks, shared, isum, osum, iexp, oexp, s); break;
        case 2: launch_s<Q, GU, 2>(a, wa, wb, xin, hout, yout, K, N, max_chunks, shared, isum, osum, iexp, oexp, s); break;
        default: launch_s<Q, GU, 1>(a, wa, wb, xin, hout, yout, K, N, max_chunks, shared, isum, osum, iexp, oexp, s); break;
    }
}

// Upper bound of the routed row chunks: every chunk holds at least one pair,
// and at most one chunk per expert is partial.
int max_routed_chunks(const FwdArgs &a) {
    return std::min(a.P, a.P / kGemvTokens + std::min(a.d.n_experts, a.P));
}

}  // namespace

// One GEMV launch of format q (run-time) on the given matrices.
template <bool GU>
void launch_q(int q, const FwdArgs &a, const uint8_t *wa, const uint8_t *wb,
              const _Float16 *xin, _Float16 *hout, float *yout, int K, int N, int max_chunks,
              int shared, const float *isum, float *osum, const int32_t *iexp, int32_t *oexp,
              hipStream_t s) {
    if (q == FW_Q4_0)
        launch<FW_Q4_0, GU>(a, wa, wb, xin, hout, yout, K, N, max_chunks, shared, nullptr,
                            nullptr, iexp, oexp, s);
    else if (q == FW_Q8_0)
        launch<FW_Q8_0, GU>(a, wa, wb, xin, hout, yout, K, N, max_chunks, shared, nullptr,
                            nullptr, iexp, oexp, s);
    else if (q == FW_Q4_K)
        launch<FW_Q4_K, GU>(a, wa, wb, xin, hout, yout, K, N, max_chunks, shared, isum, osum,
                            iexp, oexp, s);
    else if (q == FW_Q6_K)
        launch<FW_Q6_K, GU>(a, wa, wb, xin, hout, yout, K, N, max_chunks, shared, nullptr,
                            nullptr, iexp, oexp, s);
    else
        launch<FW_MXFP4, GU>(a, wa, wb, xin, hout, yout, K, N, max_chunks, shared, nullptr,
                             nullptr, iexp, oexp, s);
}

// Block sums: x rows (prepare), then h rows of the routed pairs [P][F/32]
// followed by the shared expert's [T][Fs/32].
hipError_t launch_gemv_gate_up(const FwdArgs &a, hipEvent_t routed_done, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const _Float16 *x = (const _Float16 *)(a.ws + a.L.x16);
    _Float16 *h = (_Float16 *)(a.ws + a.L.h);
    const float *xs = (const float *)(a.ws + a.L.xsum);
    float *hs = (float *)(a.ws + a.L.hsum);
    const int32_t *xe = (const int32_t *)(a.ws + a.L.xe);
    int32_t *he = (int32_t *)(a.ws + a.L.he);
    const int mc = max_routed_chunks(a);
    launch_q<true>(d.expert_q, a, a.wg, a.wu, x, h, nullptr, d.hidden, d.ffn, mc, 0, xs, hs, xe,
                   he, s);
    if (routed_done) (void)hipEventRecord(routed_done, s);
    if (d.shared_ffn > 0) {
        _Float16 *hsh = h + (size_t)a.P * d.ffn;
        float *hssh = hs + (size_t)a.P * (d.ffn / 32);
        const int sc = (a.T + kGemvTokens - 1) / kGemvTokens;
        launch_q<true>(d.shared_q, a, a.sg, a.su, x, hsh, nullptr, d.hidden, d.shared_ffn, sc, 1,
                       xs, hssh, xe, he + a.P, s);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_down(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const _Float16 *h = (const _Float16 *)(a.ws + a.L.h);
    const float *hs = (const float *)(a.ws + a.L.hsum);
    float *y = (float *)(a.ws + a.L.y);
    const int32_t *he = (const int32_t *)(a.ws + a.L.he);
    const int mc = max_routed_chunks(a);
    launch_q<false>(d.expert_q, a, a.wd, nullptr, h, nullptr, y, d.ffn, d.hidden, mc, 0, hs,
                    nullptr, he, nullptr, s);
    if (d.shared_ffn > 0) {
        const _Float16 *hsh = h + (size_t)a.P * d.ffn;
        const float *hssh = hs + (size_t)a.P * (d.ffn / 32);
        float *ysh = y + (size_t)a.P * d.hidden;
        const int sc = (a.T + kGemvTokens - 1) / kGemvTokens;
        launch_q<false>(d.shared_q, a, a.sd, nullptr, hsh, nullptr, ysh, d.shared_ffn, d.hidden,
                        sc, 1, hssh, nullptr, he + a.P, nullptr, s);
    }
    return hipGetLastError();
}

}  // namespace fw
