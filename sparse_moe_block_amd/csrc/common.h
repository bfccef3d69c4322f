// Internal declarations of the gfx950 MoE library: workspace layout, GGUF block
// decoding in registers, and the kernel launchers the C ABI calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fwmoe.h"

namespace fw {

constexpr int kWave = 64;
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;
constexpr int kUnit = 256;        // elements per 16-byte-aligned run of 8 blocks
constexpr int kGemvTokens = 8;    // tokens a GEMV lane accumulates at once
constexpr int kGemmBM = 128;      // token rows per grouped-GEMM tile
constexpr int kGemvMaxT = 64;     // AUTO: GEMV family up to this many tokens

// First 256 bytes of every workspace.
struct WsHeader {
    int32_t status;     // sticky FW_STATUS_* bits
    int32_t n_active;   // experts with at least one routed pair
    int32_t n_tiles;    // grouped-GEMM row tiles (routed experts)
    int32_t reserved[61];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

// Byte offsets of the per-call scratch areas inside the workspace.
struct WsLayout {
    size_t active;   // int32 [E + 1]                 active expert list
    size_t tiles;    // int32 [2 * max_tiles]         (expert, first row) per GEMM tile
    size_t xs;       // f32  [T][H/32]                block sums of x (GEMV)
    size_t x32;      // f32  [T][H]                   x in fp32 (GEMV)
    size_t x16;      // f16  [T][H]                   x in fp16 (GEMM)
    size_t h;        // f32  [P][F] then [T][Fs]       SiLU(g)*u (f16 in the GEMM family)
    size_t hs;       // f32  [P][F/32] then [T][Fs/32] block sums of h (GEMV)
    size_t y;        // f32  [P][H] then [T][H]        per-pair expert outputs
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
    static constexpr float kOffset = 8.0f;      // codes are decoded as q, value = d*(q-8)
};
template <> struct QT<FW_Q8_0> {
    static constexpr int kBlockBytes = 34, kUnitBytes = 272, kUnitX4 = 17;
    static constexpr float kOffset = 128.0f;    // codes are decoded as q+128, value = d*q
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

// The wavefront index inside the workgroup, as a value the compiler knows to
// be uniform across the wavefront (so loops over it stay in scalar registers).
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

// v_and_b32 the optimiser cannot narrow: keeps the four masked nibbles in byte
// lanes so that each converts with one v_cvt_f32_ubyte{0,1,2,3}.
__device__ __forceinline__ uint32_t and_opaque(uint32_t v, uint32_t m) {
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(v), "s"(m));
    return r;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
    return (float)h;
}

__device__ __forceinline__ uint32_t funnel16(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_alignbyte(hi, lo, 2);   // bytes 2..5 of hi:lo
}

// Decode block B of a unit held as dwords w[]: the fp32 scale and the 32 codes
// as floats *offset by QT<Q>::kOffset* (Q4_0: q in 0..15; Q8_0: q+128 in
// 1..255), so that value_i = d * (c_i - kOffset).
template <int Q, int B>
__device__ __forceinline__ void decode_block(const uint32_t *w, float &d, float c[32]) {
    if constexpr (Q == FW_Q4_0) {
        constexpr int base = (B / 2) * 9;  // dword index of the even block of the pair
        uint32_t q[4];
        if constexpr (B % 2 == 0) {
            d = half_bits_to_float(w[base] & 0xFFFFu);
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = funnel16(w[base + i], w[base + i + 1]);
        } else {
            d = half_bits_to_float(w[base + 4] >> 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = w[base + 5 + i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = and_opaque(q[i], 0x0F0F0F0Fu);
            const uint32_t hi = and_opaque(q[i] >> 4, 0x0F0F0F0Fu);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[4 * i + j] = (float)((lo >> (8 * j)) & 0xFFu);
                c[16 + 4 * i + j] = (float)((hi >> (8 * j)) & 0xFFu);
            }
        }
    } else {
        constexpr int base = (B / 2) * 17;
        uint32_t q[8];
        if constexpr (B % 2 == 0) {
            d = half_bits_to_float(w[base] & 0xFFFFu);
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = funnel16(w[base + i], w[base + i + 1]);
        } else {
            d = half_bits_to_float(w[base + 8] >> 16);
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = w[base + 9 + i];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t u = q[i] ^ 0x80808080u;   // signed byte q -> unsigned q + 128
#pragma unroll
            for (int j = 0; j < 4; ++j) c[4 * i + j] = (float)((u >> (8 * j)) & 0xFFu);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers (defined in the .hip files).  All enqueue on `s` and return the
// launch's hipError_t.
hipError_t launch_logits(const fw_moe_desc &d, int T, const void *x, const void *wr,
                         const float *bias, float *logits, hipStream_t s);
hipError_t launch_topk(const fw_moe_desc &d, int T, const float *logits, int32_t *ids,
                       float *w, hipStream_t s);
hipError_t launch_permute(const fw_moe_desc &d, int T, const int32_t *ids, int32_t *offsets,
                          int32_t *sorted, int32_t *inv, WsHeader *hdr, hipStream_t s);
hipError_t launch_clear_status(WsHeader *hdr, hipStream_t s);

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
hipError_t launch_gemv_gate_up(const FwdArgs &a, hipStream_t s);
hipError_t launch_gemv_down(const FwdArgs &a, hipStream_t s);
hipError_t launch_gemm_gate_up(const FwdArgs &a, hipStream_t s);
hipError_t launch_gemm_down(const FwdArgs &a, hipStream_t s);
hipError_t launch_combine(const FwdArgs &a, hipStream_t s);

}  // namespace fw
