// Weight fragments of the grouped GEMM: the fp16 MFMA B fragments (eight k
// values) dequantised in registers from a lane's window -- the dword-aligned
// bytes of two consecutive GGUF blocks of one weight row (Q4_K: the
// super-block header and one 32-byte code group).
#pragma once

#include "common.h"

namespace fw {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// Dwords of the window of blocks 2g, 2g + 1 of a unit, per weight row.
// Q4_K: the super-block's 16-byte header and the 32 code bytes of group g.
// Q6_K: 8 ql dwords (the lane group's 32 bytes of the half's low bits), 8
// qh dwords (the half's top bits, shifted right by 2g), the half's 8 scales
// (2 dwords, shifted right by 16g) and d.
// MXFP4: 8 code dwords (blocks 2g, 2g + 1 of the half) and the half's four
// scale bytes, shifted right by 16g.
template <int Q> constexpr int win_dwords() {
    return Q == FW_Q4_0 ? 9 : Q == FW_Q4_K ? 12 : Q == FW_Q6_K ? 19 : Q == FW_MXFP4 ? 9 : 17;
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

// Per-step constants of a Q6_K window, as fp32 bits: for the lane group's
// blocks k = g + 2 k2 (k2 = 0, 1), k[2 k2] = d * scale of the block's first
// 16 elements and k[2 k2 + 1] = 16 d * scale of its last 16 (their pairs
// j = 1, 3 carry 16x).  Both exact in fp32.
__device__ __forceinline__ void q6k_consts(const uint32_t *w, uint32_t *k) {
    const float d = half_bits_to_float(w[18] & 0xFFFFu);
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
        k[2 * k2] = __float_as_uint(d * (float)(int)__builtin_amdgcn_sbfe(w[16 + k2], 0, 8));
        k[2 * k2 + 1] = __float_as_uint(16.0f * d * (float)(int)__builtin_amdgcn_sbfe(w[16 + k2], 8, 8));
    }
}

// Bound on the magnitude of a Q6_K window's fp16 weights: 32 |constant|.
__device__ __forceinline__ float q6k_bound(const uint32_t *k) {
    float b = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) b = fmaxf(b, 32.0f * fabsf(__uint_as_float(k[i])));
    return b;
}

// B fragment of slice I from a Q6_K window: block k = g + 2 (I / 4) of the
// half, pairs 4 (I % 4) .. + 3.  Four six-bit codes form in the bytes of one
// dword (low bits: nibble I / 4 of the ql dword; top bits: bits 4 (I / 4) of
// the pre-shifted qh dword); each weight (q - 32) * d * scale is formed
// exactly in fp32 and rounded once to fp16 (pairs j = 1, 3 at 16x).
template <int I>
__device__ __forceinline__ h8 frag_b_q6k(const uint32_t *w, const uint32_t *k) {
    constexpr int K2 = I / 4, m = I % 4;
    const uint32_t cl = (((w[m] >> (4 * K2)) & 0x0F0F0F0Fu) |
                         (((w[8 + m] >> (4 * K2)) & 0x03030303u) << 4));
    const uint32_t chh = (((w[4 + m] >> (4 * K2)) & 0x0F0F0F0Fu) |
                          (((w[12 + m] >> (4 * K2)) & 0x03030303u) << 4));
    const float ds = __uint_as_float(k[2 * K2]), ds16 = __uint_as_float(k[2 * K2 + 1]);
    const float nds = -32.0f * ds, nds16 = -32.0f * ds16;
    auto e = [&](uint32_t v, int byte, float a, float b) {
        return (_Float16)fmaf((float)((v >> (8 * byte)) & 255u), a, b);
    };
    h8 f;
    f[0] = e(cl, 0, ds, nds);
    f[1] = e(cl, 2, ds, nds);
    f[2] = e(chh, 0, ds16, nds16);
    f[3] = e(chh, 2, ds16, nds16);
    f[4] = e(cl, 1, ds, nds);
    f[5] = e(cl, 3, ds, nds);
    f[6] = e(chh, 1, ds16, nds16);
    f[7] = e(chh, 3, ds16, nds16);
    return f;
}

// Per-step constants of an MXFP4 window: for the lane group's blocks
// b = 0, 1, k[2b] = 2^(scale_b - 127) and k[2b + 1] = 16 times that, each as
// an fp16 pair (exact: a normal or subnormal power of two while scale_b is
// 103 .. 142).  Returns the bound 96 * 2^(scale - 127) on the magnitude of
// the window's fp16 weights.
__device__ __forceinline__ float mx_consts(const uint32_t *w, uint32_t *k) {
    float b = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int e = (int)__builtin_amdgcn_ubfe(w[8], 8 * i, 8) - 127;
        const uint32_t c = __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_ldexpf(1.0f, e));
        const uint32_t c16 =
            __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_ldexpf(1.0f, e + 4));
        k[2 * i] = c | c << 16;
        k[2 * i + 1] = c16 | c16 << 16;
        b = fmaxf(b, __builtin_amdgcn_ldexpf(96.0f, e));
    }
    return b;
}

// B fragment of slice I from an MXFP4 window: block I / 4 of the lane's two,
// pairs 4 (I % 4) .. + 3.  Each pair's two nibbles (bytes 2m, 2m + 1 of the
// block's first or second 16 bytes, low nibbles for pairs j = 0, 1) become
// fp16 E2M1 / 2^14 (magnitude bits at 11..9, sign at 15), times 2^14 (the
// exact E2M1 value) and the block's power of two (x 16 for j = 1, 3): exact
// while the result stays within fp16.
template <int I>
__device__ __forceinline__ h8 frag_b_mxfp4(const uint32_t *w, const uint32_t *k) {
    constexpr int B = I / 4, m = I % 4;
    constexpr uint32_t sel = (m & 1) ? 0x0C030C02u : 0x0C010C00u;
    const uint32_t g0 = __builtin_amdgcn_perm(0u, w[4 * B + m / 2], sel);
    const uint32_t g1 = __builtin_amdgcn_perm(0u, w[4 * B + 2 + m / 2], sel);
    const h2 k14 = {(_Float16)16384.0f, (_Float16)16384.0f};
    const h2 c = as_h2(k[2 * B]), c16 = as_h2(k[2 * B + 1]);
    const h2 p0 = as_h2(((g0 << 9) & 0x0E000E00u) | ((g0 << 12) & 0x80008000u)) * k14 * c;
    const h2 p1 = as_h2(((g1 << 9) & 0x0E000E00u) | ((g1 << 12) & 0x80008000u)) * k14 * c16;
    const h2 p2 = as_h2(((g0 << 5) & 0x0E000E00u) | ((g0 << 8) & 0x80008000u)) * k14 * c;
    const h2 p3 = as_h2(((g1 << 5) & 0x0E000E00u) | ((g1 << 8) & 0x80008000u)) * k14 * c16;
    h8 f;
    f[0] = p0[0];
    f[1] = p0[1];
    f[2] = p1[0];
    f[3] = p1[1];
    f[4] = p2[0];
    f[5] = p2[1];
    f[6] = p3[0];
    f[7] = p3[1];
    return f;
}

// B fragment of slice I of any format (kq: the Q4_K / Q6_K / MXFP4 per-step constants).
template <int Q, int I>
__device__ __forceinline__ h8 frag_any(const uint32_t *w, const uint32_t *kq) {
    if constexpr (Q == FW_Q4_K)
        return frag_b_q4k<I>(w, kq);
    else if constexpr (Q == FW_Q6_K)
        return frag_b_q6k<I>(w, kq);
    else if constexpr (Q == FW_MXFP4)
        return frag_b_mxfp4<I>(w, kq);
    else
        return frag_b<Q, I>(w);
}

}  // namespace fw
