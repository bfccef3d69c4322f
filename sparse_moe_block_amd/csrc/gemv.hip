// Forward, GEMV family (decode-sized batches): dequant-fused expert projections
// that read each active expert's blocks once.  Decode is bandwidth-bound (the
// pages' runtime counts its cost in weight bytes moved per token -- Flyweight
// 0.2.0 "Quantization"), so the kernels are built around HBM streaming:
//
//  - a wavefront owns 64 consecutive weight rows of one expert and every S-th
//    256-element unit (8 GGUF blocks, 16-byte aligned) along the reduction
//    dimension; the S wavefronts of a workgroup interleave their units;
//  - weights move HBM -> LDS with global_load_lds_dwordx4 (each instruction
//    reads 1 KB of consecutive row bytes, so every cache line fetched is used
//    whole) through one buffer per wavefront (one batch in flight while the
//    previous one is consumed from registers); lane r reads row r's unit from
//    LDS (row strides of 144 / 272 bytes are bank-conflict-free for 16 lanes);
//  - codes become exact fp16 pairs in registers (decode_pairs) and meet the
//    activation pairs in v_dot2c_f32_f16 with fp32 accumulation; the fp16
//    block scale multiplies each block's partial sum once;
//  - the activations of the group's tokens are the same for every lane: they
//    are read with scalar loads and enter each dot as the scalar operand;
//  - partial sums of the S wavefronts meet in LDS and are added in wavefront
//    order, so results are deterministic.
// Gate and up rows of the same feature share a lane, so SiLU(g)*u is formed in
// registers (the fused gate/up pass that shares each activation load:
// Flyweight 0.2.0 "Current limitations").
#include <math.h>

#include "common.h"

namespace fw {
namespace {

constexpr int NT = kGemvTokens;
constexpr int kMaxSplit = 4;

typedef __attribute__((address_space(4))) const uint32_t cu32;
typedef __attribute__((address_space(3))) void lds_void;

// Stage unit u of the 64 rows starting at `tile` (row stride `rowbytes`) into
// buf[64 * X4] as [row][X4 x 16 bytes]: instruction i moves chunks
// c = 64 i + lane, chunk c being piece c % X4 of row c / X4.
template <int Q>
__device__ __forceinline__ void stage_unit(uint4 *buf, const uint8_t *tile, uint32_t rowbytes,
                                           int u, int lane) {
    constexpr int X4 = QT<Q>::kUnitX4;
#pragma unroll
    for (int i = 0; i < X4; ++i) {
        // uniform base + 32-bit lane offset: the SGPR-base addressing form
        const uint32_t c = i * kWave + lane, row = c / X4, piece = c % X4;
        const uint32_t off = row * rowbytes + (uint32_t)u * QT<Q>::kUnitBytes + piece * 16;
        __builtin_amdgcn_global_load_lds(tile + off, (lds_void *)(buf + i * kWave), 16, 0, 0);
    }
}

template <int Q>
__device__ __forceinline__ void read_unit(const uint4 *buf, int lane, uint32_t *w) {
    constexpr int X4 = QT<Q>::kUnitX4;
#pragma unroll
    for (int i = 0; i < X4; ++i) {
        const uint4 v = buf[lane * X4 + i];
        w[4 * i] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
    }
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

// acc[n] += (row's unit u) . (activation row n's unit u), n < NTK.  For up to
// two rows the next block's activations are loaded while the current block
// is consumed (two sets of 16 SGPRs per row); scheduling barriers keep one
// block's pairs live at a time.
template <int Q, int NTK>
__device__ __forceinline__ void dot_unit(const uint32_t *w, int u, cu32 *const *in,
                                         float *acc) {
    const uint32_t magic = pair_magic<Q>();
    uint32_t xa[NTK][16], xb[NTK][16];
    constexpr bool pre = NTK == 1;
    load_x<NTK>(xa, in, u, 0);
#define FW_BLOCK(B, CUR, NXT)                                       \
    if (pre && B < 7) load_x<NTK>(NXT, in, u, B + 1);              \
    else if (!pre && B > 0) load_x<NTK>(CUR, in, u, B);            \
    dot_block<Q, NTK, B>(w, CUR, magic, acc);                       \
    __builtin_amdgcn_sched_barrier(0);
    FW_BLOCK(0, xa, xb)
    FW_BLOCK(1, (pre ? xb : xa), xa)
    FW_BLOCK(2, xa, xb)
    FW_BLOCK(3, (pre ? xb : xa), xa)
    FW_BLOCK(4, xa, xb)
    FW_BLOCK(5, (pre ? xb : xa), xa)
    FW_BLOCK(6, xa, xb)
    FW_BLOCK(7, (pre ? xb : xa), xa)
#undef FW_BLOCK
}

// The units of one wave (u = wave, wave + S, ...), staged one batch at a time
// through `buf`.  A batch is read into registers, the next batch is issued
// into the same buffer, and the registers are consumed while that batch is in
// flight, so at every LDS read exactly one batch is outstanding.  With two
// matrices (gate/up) the batches alternate between them for the same unit.
// Interleaving units across the wavefronts of the workgroup makes the waves
// fetch adjacent units of the same rows together, so the cache lines two
// units share are fetched once.
template <int Q, int NV, int NTK>
__device__ __forceinline__ void stream_units(uint4 *buf, const uint8_t *ta, const uint8_t *tb,
                                             uint32_t rowbytes, int wave, int S, int U, int lane,
                                             cu32 *const *in, float (*acc)[NT]) {
    constexpr int X4 = QT<Q>::kUnitX4;
    uint32_t w[4 * X4];
    // cur accumulates the batch being consumed; with two matrices the two
    // accumulator sets swap after every batch (gate, up, gate, ...), which keeps
    // a single dot_unit in the loop body
    float cur[NTK], oth[NTK];
#pragma unroll
    for (int n = 0; n < NTK; ++n) cur[n] = oth[n] = 0.f;
    const int nb = NV * (U / S);
    stage_unit<Q>(buf, ta, rowbytes, wave, lane);
    for (int i = 0; i < nb; ++i) {
        const int u = wave + (i / NV) * S;
        read_unit<Q>(buf, lane, w);
        if (i + 1 < nb) {
            const int un = wave + ((i + 1) / NV) * S;
            stage_unit<Q>(buf, (NV == 2 && ((i + 1) & 1)) ? tb : ta, rowbytes, un, lane);
        }
        dot_unit<Q, NTK>(w, u, in, cur);
        if (NV == 2) {
#pragma unroll
            for (int n = 0; n < NTK; ++n) {
                const float t = cur[n];
                cur[n] = oth[n];
                oth[n] = t;
            }
        }
    }
    // nb is even for two matrices: cur holds gate, oth holds up
#pragma unroll
    for (int n = 0; n < NTK; ++n) {
        acc[0][n] = cur[n];
        if (NV == 2) acc[NV - 1][n] = oth[n];
    }
}

// One 64-row tile of one expert (or of the shared expert), for the expert's
// rows [rb, rb + rc) of the sorted pair list.
//  GU:  rows are gate/up features f; writes a = SiLU(W_g x) * (W_u x) as fp16
//       in pair order (the down projection's activation layout);
//  !GU: rows are outputs o; writes y = W_d a in fp32.
template <int Q, bool GU>
__global__ __launch_bounds__(kWave *kMaxSplit) void gemv_kernel(
    const uint8_t *__restrict__ wa, const uint8_t *__restrict__ wb,
    const int4 *__restrict__ active, WsHeader *__restrict__ hdr,
    const int32_t *__restrict__ sorted, const _Float16 *__restrict__ xin,
    _Float16 *__restrict__ hout, float *__restrict__ yout, int K, int N, int k, int P,
    int tiles_per_group, int shared, int shared_rows, int S) {
    constexpr int X4 = QT<Q>::kUnitX4;
    __shared__ uint4 stage[kMaxSplit][kWave * X4];
    const int g = blockIdx.x / tiles_per_group, tile = blockIdx.x % tiles_per_group;
    const size_t rowbytes = (size_t)(K / 32) * QT<Q>::kBlockBytes;
    int rb = 0, rc = shared_rows;
    const uint8_t *ta = wa, *tb = wb;
    if (!shared) {
        if (g >= ld_const(&hdr->n_active)) return;
        const int4 ex = ld_const(active + g);   // (expert, first row, rows)
        const size_t esz = (size_t)N * rowbytes;
        ta += ex.x * esz;
        if (GU) tb += ex.x * esz;
        rb = ex.y;
        rc = ex.z;
    }
    ta += (size_t)tile * kWave * rowbytes;
    if (GU) tb += (size_t)tile * kWave * rowbytes;
    const int wave = wave_id(), lane = threadIdx.x % kWave;
    uint4 *buf = stage[wave];
    const int U = K / kUnit;
    constexpr int NV = GU ? 2 : 1;
    for (int c0 = 0; c0 < rc; c0 += NT) {
        const int nt = min(NT, rc - c0);
        cu32 *in[NT];
        bool bad = false;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int r = rb + c0 + min(n, nt - 1);
            int t = r;   // the down projection reads row r of its input
            if (GU && !shared) {
                const int q = ld_const(sorted + r);
                bad |= (unsigned)q >= (unsigned)P;
                t = (unsigned)q < (unsigned)P ? q / k : 0;
            }
            in[n] = (cu32 *)(xin + (size_t)t * K);
        }
        if (bad && threadIdx.x == 0) atomicOr(&hdr->status, FW_STATUS_BAD_PAIR);
        float acc[NV][NT];
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[v][n] = 0.f;
        switch (nt) {
            case 1: stream_units<Q, NV, 1>(buf, ta, tb, rowbytes, wave, S, U, lane, in, acc); break;
            case 2: stream_units<Q, NV, 2>(buf, ta, tb, rowbytes, wave, S, U, lane, in, acc); break;
            case 3: stream_units<Q, NV, 3>(buf, ta, tb, rowbytes, wave, S, U, lane, in, acc); break;
            default: stream_units<Q, NV, 4>(buf, ta, tb, rowbytes, wave, S, U, lane, in, acc); break;
        }
        // partial sums of waves 1..S-1 meet wave 0's in LDS (their idle stage
        // buffers), added in wave order
        if (S > 1) {
            __syncthreads();
            float *red = (float *)stage[wave];
            if (wave > 0) {
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int n = 0; n < NT; ++n) red[(v * NT + n) * kWave + lane] = acc[v][n];
            }
            __syncthreads();
            if (wave == 0) {
                for (int s = 1; s < S; ++s) {
                    const float *o = (const float *)stage[s];
#pragma unroll
                    for (int v = 0; v < NV; ++v)
#pragma unroll
                        for (int n = 0; n < NT; ++n) acc[v][n] += o[(v * NT + n) * kWave + lane];
                }
            }
        }
        if (wave == 0) {
            const int row = tile * kWave + lane;
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if (n < nt) {
                    const size_t r = (size_t)(rb + c0 + n);
                    if constexpr (GU) {
                        const float gv = acc[0][n], up = acc[NV - 1][n];
                        float a = gv / (1.0f + __expf(-gv)) * up;
                        if (row & 16) a *= 0.0625f;   // pairs j = 1, 3 hold value / 16
                        hout[r * N + (row & ~31) + pair_pos(row & 31)] = (_Float16)a;
                    } else {
                        yout[r * N + row] = acc[0][n];
                    }
                }
            }
        }
        if (S > 1) __syncthreads();   // stage[] is reused by the next chunk
    }
}

// Wavefronts per workgroup: the reduction dimension is split into S ranges of
// whole 256-element units.
int pick_split(int units) {
    for (int s : {4, 3, 2})
        if (units % s == 0) return s;
    return 1;
}

template <int Q, bool GU>
void launch(const FwdArgs &a, const uint8_t *wa, const uint8_t *wb, const _Float16 *xin,
            _Float16 *hout, float *yout, int K, int N, int groups, int shared, hipStream_t s) {
    const int S = pick_split(K / kUnit), tpg = N / kWave;
    gemv_kernel<Q, GU><<<groups * tpg, kWave * S, 0, s>>>(
        wa, wb, (const int4 *)(a.ws + a.L.active), (WsHeader *)a.ws, a.sorted, xin, hout, yout,
        K, N, a.d.top_k, a.P, tpg, shared, shared ? a.T : 0, S);
}

}  // namespace

hipError_t launch_gemv_gate_up(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const _Float16 *x = (const _Float16 *)(a.ws + a.L.x16);
    _Float16 *h = (_Float16 *)(a.ws + a.L.h);
    const int groups = std::min(d.n_experts, a.P);
    if (d.expert_q == FW_Q4_0)
        launch<FW_Q4_0, true>(a, a.wg, a.wu, x, h, nullptr, d.hidden, d.ffn, groups, 0, s);
    else
        launch<FW_Q8_0, true>(a, a.wg, a.wu, x, h, nullptr, d.hidden, d.ffn, groups, 0, s);
    if (d.shared_ffn > 0) {
        _Float16 *hsh = h + (size_t)a.P * d.ffn;
        if (d.shared_q == FW_Q4_0)
            launch<FW_Q4_0, true>(a, a.sg, a.su, x, hsh, nullptr, d.hidden, d.shared_ffn, 1, 1, s);
        else
            launch<FW_Q8_0, true>(a, a.sg, a.su, x, hsh, nullptr, d.hidden, d.shared_ffn, 1, 1, s);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_down(const FwdArgs &a, hipStream_t s) {
    const fw_moe_desc &d = a.d;
    const _Float16 *h = (const _Float16 *)(a.ws + a.L.h);
    float *y = (float *)(a.ws + a.L.y);
    const int groups = std::min(d.n_experts, a.P);
    if (d.expert_q == FW_Q4_0)
        launch<FW_Q4_0, false>(a, a.wd, nullptr, h, nullptr, y, d.ffn, d.hidden, groups, 0, s);
    else
        launch<FW_Q8_0, false>(a, a.wd, nullptr, h, nullptr, y, d.ffn, d.hidden, groups, 0, s);
    if (d.shared_ffn > 0) {
        const _Float16 *hsh = h + (size_t)a.P * d.ffn;
        float *ysh = y + (size_t)a.P * d.hidden;
        if (d.shared_q == FW_Q4_0)
            launch<FW_Q4_0, false>(a, a.sd, nullptr, hsh, nullptr, ysh, d.shared_ffn, d.hidden, 1, 1, s);
        else
            launch<FW_Q8_0, false>(a, a.sd, nullptr, hsh, nullptr, ysh, d.shared_ffn, d.hidden, 1, 1, s);
    }
    return hipGetLastError();
}

}  // namespace fw
