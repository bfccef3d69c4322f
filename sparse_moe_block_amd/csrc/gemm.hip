// Forward, GEMM family (prefill-sized batches): grouped expert GEMMs on the
// 32x32x16 fp16 MFMA, weights dequantised in registers, activations fed to
// LDS by DMA.
//
// What bounds it.  Every dequantised weight fragment costs about 14 VALU
// instructions (code bits into fp16 pairs, exact, then times the block's
// fp16 scale), so the VALU work per MFMA is 14 divided by the number of
// token-row groups the fragment feeds.  Each wavefront here owns all token
// rows of its tile (four 32-row groups; five for Q4_0) and 64 weight rows
// (two 32-row groups), so a fragment feeds four or five 32x32x16 MFMAs
// (32768 flops each); the accumulators take 128 or 160 VGPRs.
//
//  - a workgroup tile is up to 128 rows (Q4_0: 160) of one expert's segment
//    of the sorted pair list (tokens gathered through sorted_pairs) times 256
//    weight rows; a tile with fewer rows runs only the 32-row groups that
//    hold rows.  An expert's rows take as few tiles as the size allows, and
//    every tile re-streams and re-dequantises the expert's weights, so the
//    fifth group saves a whole tile wherever an expert has 129-160 rows;
//  - K advances 128 elements (half a 256-element unit, four GGUF blocks) per
//    step, eight 16-wide MFMA slices.  Lane group g = lane / 32 covers blocks
//    2g and 2g + 1 of the half unit, slice s block 2g + s / 4, fp16 pairs
//    4 (s % 4) .. + 3 in the pair order of decode_pairs, on both operands (the
//    MFMA sums over k in any order);
//  - activations: the 128 x 128 fp16 tile of a step moves HBM/L2 -> LDS with
//    global_load_lds_dwordx4 (no VGPRs, no LDS store instructions), two steps
//    in flight in two LDS buffers; 16-byte chunk c of tile row r lands at
//    chunk c ^ (r % 16) of the row, so the 32 lanes that read one chunk of 32
//    rows hit distinct banks;
//  - weights: lane (n = lane % 32, g) loads the dword-aligned window of blocks
//    2g, 2g + 1 of its weight row (36 bytes Q4_0, 68 Q8_0; Q4_K: the
//    super-block header and the group's 32 code bytes) one step ahead and
//    turns one code dword into a B fragment right before its MFMAs;
//  - gate/up: a wavefront's 64 weight rows are 32 gate and the same 32 up
//    features, so a lane holds gate and up of the same (token, feature) and
//    forms SiLU(g)*u in registers; the 32 features of a wavefront are one
//    32-element block of h, stored in pair order straight from the registers;
//    the down projection's fp32 rows go straight from the accumulators too;
//  - each XCD takes a contiguous range of the row-tile list (the tiles of one
//    expert share its L2, so the expert's weights are fetched about once),
//    the ranges of about equal work (the schedule weighs each tile by its
//    row groups): under skewed routing the hottest experts' full tiles no
//    longer pile onto one XCD; consecutive workgroups of one XCD take the
//    column tiles of one row tile.
#include <math.h>

#include "common.h"
#include "gemm_frag.h"

namespace fw {
namespace {

constexpr int BK = 128;       // k per step
// token rows per tile (four or five 32-row MFMA groups) and the 16-byte
// chunks of a step's activations (2048 or 2560)
template <int Q> constexpr int tile_bm() { return gemm_tile_rows(Q); }
template <int Q> constexpr int a_chunks() { return tile_bm<Q>() * BK / 8; }
constexpr int kMaxDma = 160 * BK / 8 / 256;  // DMA instructions per thread, at most
constexpr int kMaxPX = 9;               // 16-byte weight pieces per row and half unit (Q8_0)
constexpr int kQ6PX = 10;               // Q6_K: pieces per row and half (ql 5, qh 3, tail 2)
static_assert(tile_bm<FW_Q4_0>() == 160 && tile_bm<FW_Q8_0>() == 128, "tile shapes");

typedef float f16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// Addresses are a uniform 64-bit base plus a 32-bit per-lane byte offset, the
// form the scalar-base global loads take (one VGPR per address).
struct Tile {
    const uint8_t *abase;    // activation rows (uniform)
    uint32_t aoff[kMaxDma];  // byte offsets of this thread's DMA rows, at its chunk
    const uint8_t *bbase[2]; // the expert's gate and up matrices (down: both the one)
    uint32_t woff[kMaxPX];   // byte offsets of this thread's weight pieces (unit 0, half 0)
    uint32_t wk;             // Q4_K: bit i set where piece i is a code piece (moves for half 1)
    // Q6_K (2-byte aligned units; bbase 16-byte aligned): per DMA instruction
    // i and half h, the byte offsets of the first and last byte of the
    // region its piece covers (unit 0) and the piece's offset in that region;
    // per column group, the offset of the lane's own row
    uint32_t q6s[2][kQ6PX], q6e[2][kQ6PX], q6p[kQ6PX], q6r[2];
    // MXFP4: 16-byte aligned bases of the two matrices' scales (their own
    // offset mod 16 is in the offsets) and, per column group, the offset of
    // the lane's own row's scales
    const uint8_t *sbase[2];
    uint32_t mxs[2];
    _Float16 *hout;
    float *yout;
    int ex;                  // thread tid < rows: the exponent of tile row tid
    WsHeader *hdr;
    int lane, wave, steps, rows, rb, ct, N;
};

// Weight pieces in LDS.  Each step's half unit moves to LDS by DMA in whole
// 16-byte pieces, PX per weight row (the smallest run of aligned pieces that
// covers the half; for Q4_K the 16-byte header and the half's two code
// groups): consecutive lanes take consecutive pieces of a row, a few cache
// lines per instruction.  Two half-unit buffers: the next step's half loads
// while this step's is used.
// Q6_K's half is four separate regions at a 2-byte aligned row offset: its
// 64 ql bytes (5 pieces), 32 qh bytes (3), and from its 8 scales to the
// unit's end (2): kQ6PX pieces, a region's spare pieces repeating its last.
// MXFP4's half is its 64 code bytes (4 pieces) plus the aligned piece
// holding its scales; a buffer keeps all rows' code pieces first and the
// scale pieces after them, so that every DMA instruction reads one kind.
template <int Q> constexpr int half_pieces() {
    return Q == FW_Q8_0 ? 9 : Q == FW_Q6_K ? kQ6PX : 5;
}
// source piece of LDS piece j (0 .. PX - 1) of half h of a unit
template <int Q> __device__ __forceinline__ int src_piece(int h, int j) {
    if constexpr (Q == FW_Q4_K) return h == 0 || j == 0 ? j : 4 + j;
    else return j + h * (QT<Q>::kUnitX4 - half_pieces<Q>());
}

// A lane's window of half h (blocks 2g, 2g + 1 of the half; Q4_K: the
// super-block header and code group 2h + g) from its weight row's pieces in
// LDS (row: the row's first piece).
template <int Q>
__device__ __forceinline__ void lds_window(const uint8_t *row, int h, int g, uint32_t *w,
                                           uint32_t x = 0) {
    if constexpr (Q == FW_Q6_K) {
        // x: the unit's byte offset in its first piece (= that of its ql and
        // qh halves in theirs); reads start at the dword holding a region's
        // first byte, a 2-byte offset is taken out with v_alignbyte
        const uint32_t sh = x & 3u;
        const uint32_t *ql = (const uint32_t *)(row + ((x + 32 * g) & ~3u));
        const uint32_t *qh = (const uint32_t *)(row + 80 + (x & ~3u));
        uint32_t r[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) r[i] = ql[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = __builtin_amdgcn_alignbyte(r[i + 1], r[i], sh);
#pragma unroll
        for (int i = 0; i < 9; ++i) r[i] = qh[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[8 + i] = __builtin_amdgcn_alignbyte(r[i + 1], r[i], sh) >> (2 * g);
        // scales 8h .. 8h + 7, then d 16 - 8h bytes after them
        const uint32_t t = (x + 8 * h) & 15u, st = t & 3u;
        const uint32_t *tl = (const uint32_t *)(row + 128 + (t & ~3u));
#pragma unroll
        for (int i = 0; i < 5; ++i) r[i] = tl[i];
        w[16] = __builtin_amdgcn_alignbyte(r[1], r[0], st) >> (16 * g);
        w[17] = __builtin_amdgcn_alignbyte(r[2], r[1], st) >> (16 * g);
        w[18] = h ? __builtin_amdgcn_alignbyte(r[3], r[2], st)
                  : __builtin_amdgcn_alignbyte(r[4], r[4], st);
    } else if constexpr (Q == FW_Q4_K) {
        const uint32_t *hd = (const uint32_t *)row;
        const uint32_t *cd = (const uint32_t *)(row + 16 + 32 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = hd[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[4 + i] = cd[i];
    } else {
        constexpr int kHalf = QT<Q>::kUnitBytes / 2;
        const int first = h * kHalf - 16 * src_piece<Q>(h, 0);   // 0 or 8
        const uint32_t *q = (const uint32_t *)(row + first + g * (2 * QT<Q>::kBlockBytes));
#pragma unroll
        for (int i = 0; i < win_dwords<Q>(); ++i) w[i] = q[i];
    }
}

// LDS weight row Rl of a buffer holds the workgroup's weight row Rl:
//   gate/up: Rl < 32 NW gate feature ct 32 NW + Rl, else up feature
//            ct 32 NW + Rl - 32 NW; wavefront w reads rows 32 w + n (gate)
//            and 32 NW + 32 w + n (up);
//   down:    output row ct 64 NW + Rl; wavefront w reads 64 w + 32 cg + n.
template <bool GU, int NW>
__device__ __forceinline__ int lds_wrow(int wave, int cg, int n) {
    return GU ? 32 * NW * cg + 32 * wave + n : 64 * wave + 32 * cg + n;
}

// NW wavefronts per workgroup, each owning 64 weight rows and all token rows.
template <int Q, bool GU, int NW, int MI>
__device__ __forceinline__ void tile_run(uint4 *A0, uint4 *A1, uint4 *B0, uint4 *B1,
                                          const Tile &c) {
    constexpr int kThreads = 64 * NW;
    // DMA instruction i of a thread covers tile rows [4 NW i, 4 NW (i + 1)):
    // the ones the tile's MI 32-row groups need
    constexpr int kDma = (32 * MI + 4 * NW - 1) / (4 * NW);
    constexpr int WD = win_dwords<Q>();
    constexpr int UB = QT<Q>::kUnitBytes, PX = half_pieces<Q>();
    constexpr bool kRollA = MI > 4;
    const int lane = c.lane, steps = c.steps;
    const int g = lane >> 5, n = lane & 31, wave = c.wave;

    f16v acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    uint32_t wh[2][WD];      // this step's windows, per column group
    uint32_t dmax = 0;       // largest block-scale magnitude bits met (Q8_0 / Q4_0)
    float wmax = 0.f;        // largest Q4_K weight bound met

    // activations of step st: rows 4 NW i + tid / 16, chunk (tid % 16) ^ (tid / 16 % 16)
    auto dma_a = [&](uint4 *buf, int st, int i) {
        if (i < kDma)
            __builtin_amdgcn_global_load_lds(c.abase + (c.aoff[i] + (uint32_t)st * (BK * 2)),
                                             (lds_void *)(buf + i * kThreads + 64 * wave), 16,
                                             0, 0);
    };
    // instruction i of the weight pieces of step st: LDS pieces
    // 64 (NW i + w) .. + 63 of the buffer, all of one matrix (the 32 NW rows
    // of PX pieces of each matrix are a whole number of 64-piece instructions)
    auto dma_w = [&](uint4 *buf, int st, int i) {
        if (i < PX) {
            const int h = st & 1;
            const uint8_t *base = GU && (NW * i + wave >= NW * PX / 2) ? c.bbase[1] : c.bbase[0];
            uint32_t off = 0;
            if constexpr (Q == FW_MXFP4) {
                // code pieces: rows' 64 code bytes of the half; scale
                // pieces: the aligned piece holding the unit's 8 scales
                const int j = NW * i + wave;
                const uint32_t u = (uint32_t)(st >> 1);
                if (j < 4 * NW) {
                    base = GU && j >= 2 * NW ? c.bbase[1] : c.bbase[0];
                    off = c.woff[i] + 128u * u + 64u * (uint32_t)h;
                } else {
                    base = GU && 2 * j >= 9 * NW ? c.sbase[1] : c.sbase[0];
                    off = (c.woff[i] + 8u * u) & ~15u;
                }
            } else if constexpr (Q == FW_Q6_K) {
                // the piece's aligned address, clamped to its region's last
                // piece: every piece holds a byte of its region
                const uint32_t uo = (uint32_t)(st >> 1) * UB;
                const uint32_t b0 = (h ? c.q6s[1][i] : c.q6s[0][i]) + uo;
                const uint32_t e0 = (h ? c.q6e[1][i] : c.q6e[0][i]) + uo;
                off = min((b0 & ~15u) + c.q6p[i], e0 & ~15u);
            } else {
                off = c.woff[i] + (uint32_t)(st >> 1) * UB;
                if constexpr (Q == FW_Q4_K) off += h && ((c.wk >> i) & 1) ? 64u : 0u;
                else off += (uint32_t)h * (16 * (QT<Q>::kUnitX4 - PX));
            }
            __builtin_amdgcn_global_load_lds(base + off,
                                             (lds_void *)(buf + i * kThreads + 64 * wave), 16,
                                             0, 0);
        }
    };
    const int wr0 = lds_wrow<GU, NW>(wave, 0, n) * (16 * PX);
    const int wr1 = lds_wrow<GU, NW>(wave, 1, n) * (16 * PX);
    // the windows of step st (half st % 2) from buffer buf
    auto read_w = [&](const uint4 *buf, int st) {
        const int h = st & 1;
        if constexpr (Q == FW_MXFP4) {
            // codes of LDS row Rl at 64 Rl, its scale piece at 16 (256 NW + Rl)
#pragma unroll
            for (int cg = 0; cg < 2; ++cg) {
                const int Rl = lds_wrow<GU, NW>(wave, cg, n);
                const uint4 *cd = (const uint4 *)((const uint8_t *)buf + 64 * Rl + 32 * g);
                const uint4 q0 = cd[0], q1 = cd[1];
                wh[cg][0] = q0.x; wh[cg][1] = q0.y; wh[cg][2] = q0.z; wh[cg][3] = q0.w;
                wh[cg][4] = q1.x; wh[cg][5] = q1.y; wh[cg][6] = q1.z; wh[cg][7] = q1.w;
                const uint32_t sub = (c.mxs[cg] + 8u * (uint32_t)(st >> 1)) & 15u;
                wh[cg][8] = *(const uint32_t *)((const uint8_t *)buf + 16 * (256 * NW + Rl) +
                                                sub + 4 * h) >> (16 * g);
            }
        } else if constexpr (Q == FW_Q6_K) {
            const uint32_t uo = (uint32_t)(st >> 1) * UB;
            lds_window<Q>((const uint8_t *)buf + wr0, h, g, wh[0], (c.q6r[0] + uo) & 15u);
            lds_window<Q>((const uint8_t *)buf + wr1, h, g, wh[1], (c.q6r[1] + uo) & 15u);
        } else {
            lds_window<Q>((const uint8_t *)buf + wr0, h, g, wh[0]);
            lds_window<Q>((const uint8_t *)buf + wr1, h, g, wh[1]);
        }
    };
    // A fragment of slice s, row group mi: row 32 mi + n, chunk 8 g + s (Q6_K:
    // 4 g + 8 (s / 4) + s % 4, the lane group's blocks being g and g + 2),
    // stored at the chunk's index ^ (n % 16) in the row
    const int arow = n * 16, ax = n & 15;
    constexpr int kGC = Q == FW_Q6_K ? 4 : 8;
    auto apos = [&](int S) {
        const int cs = Q == FW_Q6_K ? 8 * (S >> 2) + (S & 3) : S;
        return arow + ((kGC * g + cs) ^ ax);
    };
    // One step: eight slices, software-pipelined one slice deep -- slice S's
    // MFMAs are issued with slice S + 1's A fragments already on their way
    // from LDS and followed by slice S + 1's B fragments, so a wavefront's
    // MFMAs run back to back without waiting on its own LDS reads or dequant.
    // pf(S) issues the DMA instructions placed after slice S.
    auto step = [&](const uint4 *buf, int h, auto &&pf) {
        uint32_t kq[2][4];
        if constexpr (Q == FW_Q4_K) {
#pragma unroll
            for (int cg = 0; cg < 2; ++cg) {
                q4k_consts(wh[cg], 2 * h + g, kq[cg]);
                wmax = fmaxf(wmax, q4k_bound(kq[cg]));
            }
        } else if constexpr (Q == FW_Q6_K) {
#pragma unroll
            for (int cg = 0; cg < 2; ++cg) {
                q6k_consts(wh[cg], kq[cg]);
                wmax = fmaxf(wmax, q6k_bound(kq[cg]));
            }
        } else if constexpr (Q == FW_MXFP4) {
#pragma unroll
            for (int cg = 0; cg < 2; ++cg) wmax = fmaxf(wmax, mx_consts(wh[cg], kq[cg]));
        } else {
#pragma unroll
            for (int cg = 0; cg < 2; ++cg) dmax = max(dmax, d_bits<Q>(wh[cg]));
        }
        h8 a[2][MI], b[2][2];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) a[0][mi] = __builtin_bit_cast(h8, buf[apos(0) + mi * 512]);
        b[0][0] = frag_any<Q, 0>(wh[0], kq[0]);
        b[0][1] = frag_any<Q, 0>(wh[1], kq[1]);
        // Five row groups (160 accumulators) leave no registers for a second
        // set of A fragments: there each group's next-slice fragment is read
        // into its own registers right after the group's two MFMAs, and is
        // waited on a slice later, behind the other groups' MFMAs.
#define FW_SLICE(S)                                                                          \
    {                                                                                        \
        constexpr int X = (S) & 1, Y = X ^ 1;                                                \
        if constexpr (kRollA) {                                                              \
            _Pragma("unroll") for (int mi = 0; mi < MI; ++mi) {                              \
                _Pragma("unroll") for (int cg = 0; cg < 2; ++cg)                             \
                    acc[mi][cg] = __builtin_amdgcn_mfma_f32_32x32x16_f16(                    \
                        a[0][mi], b[X][cg], acc[mi][cg], 0, 0, 0);                           \
                if constexpr ((S) < 7)                                                       \
                    a[0][mi] = __builtin_bit_cast(h8, buf[apos((S) + 1) + mi * 512]);        \
            }                                                                                \
        } else {                                                                             \
            if constexpr ((S) < 7) {                                                         \
                _Pragma("unroll") for (int mi = 0; mi < MI; ++mi)                            \
                    a[Y][mi] = __builtin_bit_cast(h8, buf[apos((S) + 1) + mi * 512]);        \
            }                                                                                \
            _Pragma("unroll") for (int cg = 0; cg < 2; ++cg)                                 \
                _Pragma("unroll") for (int mi = 0; mi < MI; ++mi)                            \
                    acc[mi][cg] = __builtin_amdgcn_mfma_f32_32x32x16_f16(                    \
                        a[X][mi], b[X][cg], acc[mi][cg], 0, 0, 0);                           \
        }                                                                                    \
        if constexpr ((S) < 7) {                                                             \
            b[Y][0] = frag_any<Q, ((S) + 1) & 7>(wh[0], kq[0]);                              \
            b[Y][1] = frag_any<Q, ((S) + 1) & 7>(wh[1], kq[1]);                              \
        }                                                                                    \
        pf(S);                                                                               \
        __builtin_amdgcn_sched_barrier(0);                                                   \
    }
        FW_SLICE(0)
        FW_SLICE(1)
        FW_SLICE(2)
        FW_SLICE(3)
        FW_SLICE(4)
        FW_SLICE(5)
        FW_SLICE(6)
        FW_SLICE(7)
#undef FW_SLICE
    };
    // sync: everything issued so far has landed (one full wait, as a builtin
    // so the compiler's own wait insertion knows of it) and every wavefront
    // has reached the same point, so a buffer read before it may be refilled
    // after it.  The loop body has no branch (the compiler's tracking of
    // which LDS buffer a pending DMA writes does not survive one): past the
    // last step the prefetches repeat the last step's addresses.
    auto sync = [&]() {
        __builtin_amdgcn_s_waitcnt(7 << 4);   // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // Step st reads activations A[st % 2] and weights B[st % 2] and loads
    // step st + 1's into the other pair of buffers, which every wavefront
    // finished reading before the sync that ended step st - 1.  The DMA
    // instructions follow the first slices rather than all come at the
    // step's start: a burst of every wavefront's DMA fills the memory
    // pipeline's queues and holds up the MFMAs behind it.
    auto issue = [&](uint4 *abuf, uint4 *bbuf, int st, int S) {
        if (S < 4) {
#pragma unroll
            for (int i = 0; i < (PX + 3) / 4; ++i) dma_w(bbuf, st, S * ((PX + 3) / 4) + i);
        }
        if (S < 2) {
#pragma unroll
            for (int i = 0; i < (kDma + 1) / 2; ++i) dma_a(abuf, st, S * ((kDma + 1) / 2) + i);
        }
    };
#pragma unroll
    for (int i = 0; i < PX; ++i) dma_w(B0, 0, i);
#pragma unroll
    for (int i = 0; i < kDma; ++i) dma_a(A0, 0, i);
    sync();
    for (int st = 0; st < steps; st += 2) {
        read_w(B0, st);
        step(A0, 0, [&](int S) { issue(A1, B1, st + 1, S); });
        sync();
        read_w(B1, st + 1);
        const int nx = min(st + 2, steps - 1);
        step(A1, 1, [&](int S) { issue(A0, B0, nx, S); });
        sync();
    }

    // ---- epilogue: acc[mi][cg][v] is tile row 32 mi + 8 (v / 4) + 4 g + v % 4,
    // weight row (column group cg) n ----
    const int rows = c.rows, rb = c.rb, N = c.N;
    // each tile row's exponent, through LDS: the activation buffers are free
    // once the last step's sync has passed
    int32_t *s_ex = (int32_t *)A1;
    if ((int)threadIdx.x < rows) s_ex[threadIdx.x] = c.ex;
    __syncthreads();
    bool range = (Q == FW_Q4_K || Q == FW_Q6_K || Q == FW_MXFP4)
                     ? !(wmax <= 65504.0f)
                     : dmax > (Q == FW_Q4_0 ? kQ4DMaxBits : kQ8DMaxBits);
    if constexpr (GU) {
        // feature ct * 128 + 32 wave + n: gate in column group 0, up in 1; the
        // wavefront's 32 features are one 32-element block of h (pair order)
        _Float16 *hrow = c.hout + (size_t)c.ct * (32 * NW) + 32 * c.wave + pair_pos(n);
        const int esc = (n & 16) ? 4 : 0;   // pairs j = 1, 3 hold value / 16
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 32 * mi + 8 * (v >> 2) + 4 * g + (v & 3);
                if (row < rows) {
                    const int e = s_ex[row];
                    const float gv = __builtin_amdgcn_ldexpf(acc[mi][0][v], -e);
                    const float up = __builtin_amdgcn_ldexpf(acc[mi][1][v], -e);
                    const float a = gv / (1.0f + __expf(-gv)) * up;
                    const _Float16 ah = (_Float16)__builtin_amdgcn_ldexpf(a, 2 * e - esc);
                    range |= (__builtin_bit_cast(uint16_t, ah) & 0x7C00u) == 0x7C00u;
                    hrow[(size_t)(rb + row) * N] = ah;
                }
            }
    } else {
        // y rows at the row's scale: for each (mi, cg, v) the 32 lanes of a
        // lane group write 128 contiguous bytes of one row
        float *yrow = c.yout + (size_t)c.ct * (64 * NW) + 64 * c.wave + n;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 32 * mi + 8 * (v >> 2) + 4 * g + (v & 3);
                if (row < rows) {
                    const int e = s_ex[row];
#pragma unroll
                    for (int cg = 0; cg < 2; ++cg)
                        yrow[(size_t)(rb + row) * N + 32 * cg] =
                            __builtin_amdgcn_ldexpf(acc[mi][cg][v], -e);
                }
            }
    }
    if (range) atomicOr(&c.hdr->status, FW_STATUS_RANGE);
}

// One (row tile, column tile) of one expert (or of the shared expert).
//  GU:  A = x rows gathered through sorted_pairs (routed) or token rows
//       (shared); weight rows = 128 gate + 128 up features; writes
//       a = SiLU(g) * u (fp16, pair order, at 2^(2e)) for 128 features and
//       each h row's exponent 2e (oexp);
//  !GU: A = rows of a (fp16); weight rows = 256 outputs; writes y (fp32)
//       scaled back by the h row's exponent (iexp).
// Two half-unit weight buffers (64 NW rows) and two activation tiles (64 KB)
// fill most of a CU's 160 KB, so one workgroup runs per CU.  Eight-wave workgroups
// (two wavefronts per SIMD, within 256 registers) serve Q4_0 and Q4_K;
// four-wave ones (one wavefront per SIMD, up to 512 registers) serve the
// column counts eight waves do not divide and Q8_0, whose wider windows and
// 272-byte units need the registers and the LDS.
template <int Q, int NW> constexpr int waves_per_simd() { return NW == 8 ? 2 : 1; }
template <int Q> constexpr bool eight_waves() {
    return Q == FW_Q4_0 || Q == FW_Q4_K || Q == FW_MXFP4;
}

template <int Q, bool GU, int NW>
__global__ __launch_bounds__(64 * NW, (waves_per_simd<Q, NW>() * 4 / NW)) void gemm_kernel(
    const uint8_t *__restrict__ wa, const uint8_t *__restrict__ wb,
    const int4 *__restrict__ tiles, WsHeader *__restrict__ hdr,
    const int32_t *__restrict__ sorted, const _Float16 *__restrict__ ain,
    _Float16 *__restrict__ hout, float *__restrict__ yout, int K, int N, int k, int P,
    int col_tiles, int n_row_tiles_max, int shared, int shared_rows,
    const int32_t *__restrict__ iexp, int32_t *__restrict__ oexp, size_t sreg) {
    constexpr int PX = half_pieces<Q>();
    constexpr int BM = tile_bm<Q>();
    __shared__ uint4 A0[a_chunks<Q>()];
    __shared__ uint4 A1[a_chunks<Q>()];
    __shared__ uint4 B0[64 * NW * PX];   // half units of the workgroup's weight rows
    __shared__ uint4 B1[64 * NW * PX];
    // XCD-aware order (the tiles of one expert are consecutive)
    int ct;
    const int rt = xcd_row_tile(hdr, col_tiles, n_row_tiles_max, shared,
                                (shared_rows + BM - 1) / BM, ct);
    if (rt < 0) return;
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
    constexpr int kThreads = 64 * NW;
    const int tid = threadIdx.x;
    // each row's source row (the token of a routed gate/up row) and exponent
    auto src_row = [&](int r) {   // r < rows
        if (GU && !shared) {
            const int q = sorted[rb + r];
            if ((unsigned)q >= (unsigned)P) {
                atomicOr(&hdr->status, FW_STATUS_BAD_PAIR);
                return 0;
            }
            return q / k;
        }
        return rb + r;
    };
    // the exponent of tile row tid: its token's x exponent (gate/up) or the
    // h row's (down)
    int ex = 0;
    if (tid < rows) {
        ex = iexp[src_row(tid)];
        if (GU && ct == 0) oexp[rb + tid] = 2 * ex;
    }
    Tile c;
    c.ex = ex;
    c.lane = tid % kWave;
    c.wave = wave_id();
    // DMA rows 4 NW i + tid / 16 (past the tile's end: its last row), chunk
    // (tid % 16) ^ (tid / 16 % 16), as byte offsets into ain
    const int chunk = (tid & 15) ^ ((tid >> 4) & 15);
#pragma unroll
    for (int i = 0; i < a_chunks<Q>() / kThreads; ++i) {
        const int r = min(4 * NW * i + (tid >> 4), rows - 1);
        int s = rb + r;
        if (GU && !shared) {
            const int q = sorted[s];
            s = (unsigned)q < (unsigned)P ? q / k : 0;
        }
        c.aoff[i] = ((uint32_t)s * K + chunk * 8) * 2;
    }
    c.abase = (const uint8_t *)ain;
    const size_t rowbytes = QT<Q>::row_bytes(K);
    const size_t esz = (size_t)N * rowbytes;
    const uint8_t *ba = wa + (size_t)expert * esz, *bb = (GU ? wb : wa) + (size_t)expert * esz;
    // weight piece of DMA instruction i: LDS piece p = i kThreads + tid is
    // piece p % PX of LDS row p / PX (gate/up: rows from 32 NW on are the up
    // matrix's, read from bbase[1])
    if constexpr (Q == FW_MXFP4) {
        // codes: the expert's matrix rows of K / 2 bytes; scales: rows of
        // K / 32 bytes from sreg bytes into each matrix
        c.bbase[0] = ba;
        c.bbase[1] = bb;
        const uint8_t *sa0 = wa + sreg + (size_t)expert * N * (K / 32);
        const uint8_t *sb0 = (GU ? wb : wa) + sreg + (size_t)expert * N * (K / 32);
        const uint32_t smis[2] = {(uint32_t)(uintptr_t)sa0 & 15u, (uint32_t)(uintptr_t)sb0 & 15u};
        c.sbase[0] = sa0 - smis[0];
        c.sbase[1] = sb0 - smis[1];
#pragma unroll
        for (int i = 0; i < PX; ++i) {
            const int p = i * kThreads + tid;
            int Rl, m = 0;
            uint32_t piece = 0;
            const bool code = p < 256 * NW;
            if (code) {
                Rl = p / 4;
                piece = p % 4;
            } else {
                Rl = p - 256 * NW;
            }
            if (GU && Rl >= 32 * NW) {
                Rl -= 32 * NW;
                m = 1;
            }
            const int row = GU ? ct * (32 * NW) + Rl : ct * (64 * NW) + Rl;
            c.woff[i] = code ? (uint32_t)row * (uint32_t)(K / 2) + 16u * piece
                             : smis[m] + (uint32_t)row * (uint32_t)(K / 32);
        }
        const int n = c.lane & 31;
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
            const int row = GU ? ct * (32 * NW) + 32 * c.wave + n
                               : ct * (64 * NW) + 64 * c.wave + 32 * cg + n;
            c.mxs[cg] = smis[GU ? cg : 0] + (uint32_t)row * (uint32_t)(K / 32);
        }
    } else if constexpr (Q == FW_Q6_K) {
        // 16-byte aligned bases; offsets carry the matrices' own misalignment
        const uint32_t mis[2] = {(uint32_t)(uintptr_t)ba & 15u, (uint32_t)(uintptr_t)bb & 15u};
        c.bbase[0] = ba - mis[0];
        c.bbase[1] = bb - mis[1];
#pragma unroll
        for (int i = 0; i < PX; ++i) {
            const int p = i * kThreads + tid;
            int Rl = p / PX;
            const int j = p - Rl * PX;
            int m = 0;
            if (GU && Rl >= 32 * NW) {
                Rl -= 32 * NW;
                m = 1;
            }
            const int row = GU ? ct * (32 * NW) + Rl : ct * (64 * NW) + Rl;
            const uint32_t ro = mis[m] + (uint32_t)(row * rowbytes);
            // regions: ql half [64h, 64h + 64), qh half [128 + 32h, + 32),
            // scales of the half to the unit's end [192 + 8h, 210)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t b0 = j < 5 ? 64 * h : j < 8 ? 128 + 32 * h : 192 + 8 * h;
                const uint32_t e0 = j < 5 ? 64 * h + 63 : j < 8 ? 159 + 32 * h : 209;
                c.q6s[h][i] = ro + b0;
                c.q6e[h][i] = ro + e0;
            }
            c.q6p[i] = 16u * (uint32_t)(j < 5 ? j : j < 8 ? j - 5 : j - 8);
        }
        // the rows this lane reads windows of (lds_wrow)
        const int n = c.lane & 31;
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
            const int row = GU ? ct * (32 * NW) + 32 * c.wave + n
                               : ct * (64 * NW) + 64 * c.wave + 32 * cg + n;
            c.q6r[cg] = mis[GU ? cg : 0] + (uint32_t)(row * rowbytes);
        }
    } else {
        c.bbase[0] = ba;
        c.bbase[1] = bb;
        c.wk = 0;
#pragma unroll
        for (int i = 0; i < PX; ++i) {
            const int p = i * kThreads + tid;
            int Rl = p / PX;
            const int j = p - Rl * PX;
            if (GU && Rl >= 32 * NW) Rl -= 32 * NW;
            const int row = GU ? ct * (32 * NW) + Rl : ct * (64 * NW) + Rl;
            c.woff[i] = (uint32_t)(row * rowbytes) + (uint32_t)j * 16;
            if (j > 0) c.wk |= 1u << i;
        }
    }
    c.hout = hout;
    c.yout = yout;
    c.hdr = hdr;
    c.steps = K / BK;
    c.rows = rows;
    c.rb = rb;
    c.ct = ct;
    c.N = N;
    // only the 32-row groups that hold rows of this tile run
    const int mi = (rows + 31) / 32;
    if (BM > 128 && mi > 4) tile_run<Q, GU, NW, BM / 32>(A0, A1, B0, B1, c);
    else if (mi > 3) tile_run<Q, GU, NW, 4>(A0, A1, B0, B1, c);
    else if (mi > 2) tile_run<Q, GU, NW, 3>(A0, A1, B0, B1, c);
    else if (mi > 1) tile_run<Q, GU, NW, 2>(A0, A1, B0, B1, c);
    else tile_run<Q, GU, NW, 1>(A0, A1, B0, B1, c);
}

template <int Q, bool GU, int NW>
void launch_nw(const FwdArgs &a, const uint8_t *wa, const uint8_t *wb, const _Float16 *ain,
                _Float16 *hout, float *yout, int K, int N, int shared, const int32_t *iexp,
                int32_t *oexp, hipStream_t s) {
    const int col_tiles = GU ? N / (32 * NW) : N / (64 * NW);
    // routed: at most one partial tile per expert
    constexpr int BM = tile_bm<Q>();
    const int row_tiles = shared ? (a.T + BM - 1) / BM
                                 : gemm_row_tiles(a.P, a.d.n_experts, BM, a.L.max_tiles);
    const int nblk = (row_tiles + 7) / 8 * 8 * col_tiles;   // eight XCDs x whole row tiles
    gemm_kernel<Q, GU, NW><<<nblk, 64 * NW, 0, s>>>(
        wa, wb, (const int4 *)(a.ws + a.L.tiles), (WsHeader *)a.ws, a.sorted, ain, hout, yout,
        K, N, a.d.top_k, a.P, col_tiles, row_tiles, shared, shared ? a.T : 0, iexp, oexp,
        (size_t)(shared ? 1 : a.d.n_experts) * N * (size_t)(K / 2));
}

// Eight-wave workgroups wherever the format allows and the columns divide
// (gate/up: 256 features, down: 512 output rows per workgroup).
template <int Q, bool GU>
void launch(const FwdArgs &a, const uint8_t *wa, const uint8_t *wb, const _Float16 *ain,
             _Float16 *hout, float *yout, int K, int N, int shared, const int32_t *iexp,
             int32_t *oexp, hipStream_t s) {
    if constexpr (eight_waves<Q>()) {
        if (N % (GU ? 256 : 512) == 0) {
            launch_nw<Q, GU, 8>(a, wa, wb, ain, hout, yout, K, N, shared, iexp, oexp, s);
            return;
        }
    }
    launch_nw<Q, GU, 4>(a, wa, wb, ain, hout, yout, K, N, shared, iexp, oexp, s);
}

template <bool GU>
void launch_q(int q, const FwdArgs &a, const uint8_t *wa, const uint8_t *wb,
               const _Float16 *ain, _Float16 *hout, float *yout, int K, int N, int shared,
               const int32_t *iexp, int32_t *oexp, hipStream_t s) {
    if (q == FW_Q4_0)
        launch<FW_Q4_0, GU>(a, wa, wb, ain, hout, yout, K, N, shared, iexp, oexp, s);
    else if (q == FW_Q4_K)
        launch<FW_Q4_K, GU>(a, wa, wb, ain, hout, yout, K, N, shared, iexp, oexp, s);
    else if (q == FW_Q6_K)
        launch<FW_Q6_K, GU>(a, wa, wb, ain, hout, yout, K, N, shared, iexp, oexp, s);
    else if (q == FW_MXFP4)
        launch<FW_MXFP4, GU>(a, wa, wb, ain, hout, yout, K, N, shared, iexp, oexp, s);
    else
        launch<FW_Q8_0, GU>(a, wa, wb, ain, hout, yout, K, N, shared, iexp, oexp, s);
}

}  // namespace

hipError_t launch_gemm_gate_up(const FwdArgs &a, hipEvent_t routed_done, hipStream_t s) {
    if (a.d.act_quant == FW_ACT_MXFP8) return launch_gemm_mx_gate_up(a, routed_done, s);
    if (a.d.act_quant == FW_ACT_INT8) return launch_gemm_i8_gate_up(a, routed_done, s);
    const fw_moe_desc &d = a.d;
    const _Float16 *x = (const _Float16 *)(a.ws + a.L.x16);
    _Float16 *h = (_Float16 *)(a.ws + a.L.h);
    const int32_t *xe = (const int32_t *)(a.ws + a.L.xe);
    int32_t *he = (int32_t *)(a.ws + a.L.he);
    launch_q<true>(d.expert_q, a, a.wg, a.wu, x, h, nullptr, d.hidden, d.ffn, 0, xe, he, s);
    if (routed_done) (void)hipEventRecord(routed_done, s);
    if (d.shared_ffn > 0)
        launch_q<true>(d.shared_q, a, a.sg, a.su, x, h + (size_t)a.P * d.ffn, nullptr, d.hidden,
                        d.shared_ffn, 1, xe, he + a.P, s);
    return hipGetLastError();
}

hipError_t launch_gemm_down(const FwdArgs &a, hipStream_t s) {
    if (a.d.act_quant == FW_ACT_MXFP8) return launch_gemm_mx_down(a, s);
    if (a.d.act_quant == FW_ACT_INT8) return launch_gemm_i8_down(a, s);
    const fw_moe_desc &d = a.d;
    const _Float16 *h = (const _Float16 *)(a.ws + a.L.h);
    float *y = (float *)(a.ws + a.L.y);
    const int32_t *he = (const int32_t *)(a.ws + a.L.he);
    launch_q<false>(d.expert_q, a, a.wd, nullptr, h, nullptr, y, d.ffn, d.hidden, 0, he,
                     nullptr, s);
    if (d.shared_ffn > 0)
        launch_q<false>(d.shared_q, a, a.sd, nullptr, h + (size_t)a.P * d.ffn, nullptr,
                         y + (size_t)a.P * d.hidden, d.shared_ffn, d.hidden, 1, he + a.P,
                         nullptr, s);
    return hipGetLastError();
}

}  // namespace fw
