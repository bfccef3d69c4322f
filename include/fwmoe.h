/*
 * fwmoe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts FFN layer
 * run directly on GGUF block-quantised expert weights.
 *
 * The layer is the "sparse MoE execution" with grouped routed-expert GPU
 * kernels per weight format that Flyweight describes (Flyweight 0.2.0 wheel
 * METADATA, "Features" and "Quantization"; Flyweight 0.5.1, "Models and
 * formats", which lists Q4_0 and Q8_0 among the formats with grouped
 * routed-expert GPU kernels).  Its steps:
 *
 *   fw_moe_route    router logits, softmax or sigmoid scores, top-k selection,
 *                   renormalised gate weights;
 *   fw_moe_permute  token -> expert grouping (expert-sorted pair lists);
 *   fw_moe_forward  per expert: block dequant fused into the gate/up
 *                   projections, SiLU(gate)*up, dequant-fused down projection;
 *                   then the per-token weighted combine (+ shared expert).
 *
 * Conventions shared by every entry point
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except
 *    `desc` (host) and the host out-argument of fw_moe_read_status.  The
 *    library allocates nothing, keeps no pointer after returning, and never
 *    waits on the host: work is enqueued on `stream` (a hipStream_t; NULL is
 *    the null stream) and the caller keeps every buffer alive until the stream
 *    has passed it.  No entry point other than fw_moe_read_status synchronises,
 *    so route -> permute -> forward can be captured in one hipGraph.  (The
 *    pages' runtime keeps host synchronisation points inside dynamic MoE
 *    routing -- Flyweight 0.2.0, "Current limitations" -- this ABI has none.)
 *  - Row-major everywhere.  Device pointers must be 16-byte aligned and the
 *    workspace 256-byte aligned.
 *  - Arguments are validated before anything is enqueued: a negative return
 *    means nothing was launched.  Unsupported requests are refused with
 *    FW_EUNSUPPORTED, never served by a slower fallback (the pages' own rule of
 *    refusing rather than silently not engaging, Flyweight 0.2.0
 *    "Quantization").
 *  - Data-dependent errors found on the device (an expert id outside [0, E), an
 *    offset or pair index out of range) never fault: the offending pair is
 *    skipped and a sticky bit is OR-ed into the status word at the start of the
 *    workspace.  fw_moe_read_status reads it; fw_moe_clear_status resets it.
 *  - Results are deterministic: repeated calls on the same inputs are bitwise
 *    identical (no floating-point atomics; fixed summation orders).
 *  - Stateless and thread-safe: the library keeps no state between calls
 *    beyond per-device properties it queries once (CU count, kernel
 *    occupancy); calls from several host threads on their own streams and
 *    workspaces do not interfere.
 *
 * GGUF block layouts (the pages name the formats but print no byte layout; the
 * layout is GGUF's, little-endian, no padding):
 *   Q8_0: [fp16 d][32 x int8 q]                 34 bytes, value = d * q
 *   Q4_0: [fp16 d][16 bytes]                    18 bytes, value = d * (q - 8),
 *         byte i holds element i (low nibble) and element i+16 (high nibble).
 * Expert tensors are blocked along the reduction dimension of each projection:
 *   w_gate, w_up : [E][F][H/32 blocks]   row f of expert e reads x (length H)
 *   w_down       : [E][H][F/32 blocks]   row o of expert e reads the F-vector
 * and the shared expert's tensors are the same without the leading [E].
 */
#ifndef FWMOE_H
#define FWMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
    FW_OK = 0,
    FW_EINVAL = -1,        /* bad size, null pointer or out-of-range enum   */
    FW_EUNSUPPORTED = -2,  /* a combination this library does not serve     */
    FW_EWORKSPACE = -3,    /* workspace missing or smaller than required    */
    FW_EALIGN = -4,        /* a pointer is not 16-byte (workspace: 256) aligned */
    FW_EHIP = -5           /* the HIP runtime reported an error on launch   */
};

/* Device status bits (sticky, in the workspace's status word). */
enum {
    FW_STATUS_BAD_EXPERT_ID = 1, /* fw_moe_permute met an id outside [0, E)      */
    FW_STATUS_BAD_OFFSETS = 2,   /* fw_moe_forward met non-monotone / out-of-range
                                    expert_offsets (clamped)                     */
    FW_STATUS_BAD_PAIR = 4,      /* fw_moe_forward met a sorted_pairs / inv_pos
                                    entry out of range (skipped)                 */
    FW_STATUS_RANGE = 8          /* fw_moe_forward met a value its fp16 operands
                                    cannot hold: a non-finite activation, a
                                    SwiGLU output beyond +-65504 after the
                                    per-token scaling, or (grouped GEMM) a block
                                    scale whose dequantised codes exceed fp16;
                                    the affected outputs are not reliable       */
};

enum { FW_F32 = 0, FW_BF16 = 1 };                 /* activation / router dtype */
enum { FW_Q8_0 = 0, FW_Q4_0 = 1, FW_Q4_K = 2, FW_Q6_K = 3, FW_MXFP4 = 4 };  /* weight format */
enum { FW_SOFTMAX_RENORM = 0, FW_SIGMOID_RENORM = 1 };
enum { FW_PATH_AUTO = 0, FW_PATH_GEMV = 1, FW_PATH_GEMM = 2 };
/* Expert activations: as handed in (fp16 staging, exact for bf16 inputs in
 * range), or MXFP8 -- the MX alternative beside MXFP4 experts (vOOM, the lossy
 * artifact notes: MX formats of group size 32, MXFP8 as the control).  With
 * FW_ACT_MXFP8 each expert's input (x, and the SwiGLU output before the down
 * projection) is quantised per 32 consecutive values by the OCP MX rule
 * (scale 2^(floor(log2 amax) - 8), E4M3 elements nearest-even, clamped at
 * 448) and the expert GEMMs run on the block-scaled MFMA (E4M3 x E2M1, no
 * weight dequantisation).  Requires MXFP4 experts (and an MXFP4 shared expert
 * if any) and the grouped-GEMM family: FW_PATH_GEMV is FW_EUNSUPPORTED and
 * AUTO takes FW_PATH_GEMM for every T.  Routing uses x as handed in.
 * FW_ACT_INT8 is the int8-activation path of the pages' MMQ kernels (Flyweight
 * 0.2.0 wheel METADATA: "Runtime controls", prompt processing's routed experts
 * on block-table MMQ kernels; "Image generation", activations quantised to
 * int8 for them): each expert's input is quantised per 32 consecutive values
 * as GGUF's Q8_1-style block (d = fp32(amax / 127), codes round(fp32(v / d))
 * with halves away from zero, d kept in fp32) and the expert GEMMs run on the
 * int8 MFMA, one 32-element weight block per instruction, the scales d_x d_w
 * applied to its int32 sums in fp32.  Requires Q8_0 or Q4_0 experts (and
 * shared expert, if any) and the grouped-GEMM family, as FW_ACT_MXFP8 does. */
enum { FW_ACT_NONE = 0, FW_ACT_MXFP8 = 1, FW_ACT_INT8 = 2 };

/* Shape and formats of one MoE layer.  All fields are int32. */
typedef struct {
    int32_t hidden;       /* H: multiple of 256, 256..16384                        */
    int32_t n_experts;    /* E: 1..512                                             */
    int32_t top_k;        /* k: 1..min(E, 16)                                      */
    int32_t ffn;          /* F: routed expert inner size, multiple of 256, <= 16384 */
    int32_t shared_ffn;   /* Fs: 0 = no shared expert, else multiple of 256        */
    int32_t act_dtype;    /* FW_F32 | FW_BF16: x                                   */
    int32_t router_dtype; /* FW_F32 | FW_BF16: router weights; must equal act_dtype */
    int32_t expert_q;     /* FW_Q8_0 | FW_Q4_0 | FW_Q4_K | FW_Q6_K | FW_MXFP4       */
    int32_t shared_q;     /* same choices: shared expert (ignored if Fs = 0)      */
    int32_t score;        /* FW_SOFTMAX_RENORM | FW_SIGMOID_RENORM                 */
    int32_t path;         /* FW_PATH_*: forward kernel family (AUTO picks by T)    */
    int32_t act_quant;    /* FW_ACT_NONE | FW_ACT_MXFP8 | FW_ACT_INT8: expert inputs */
} fw_moe_desc;

/* Library version string. */
const char *fw_moe_version(void);

/* Check a descriptor; FW_OK or the reason it is refused. */
int fw_moe_validate(const fw_moe_desc *desc);

/* Bytes of workspace fw_moe_permute / fw_moe_forward need for up to max_T
 * tokens; 0 if the descriptor is invalid or max_T < 0.  The same workspace may
 * serve both calls (and any T <= max_T). */
size_t fw_moe_workspace_size(const fw_moe_desc *desc, int32_t max_T);

/* Router: logits, scores, top-k, renormalised gate weights.
 * (Flyweight 0.2.0, served-families table: "DeepSeek-shaped MoE" -> sigmoid
 * scores; vOOM notes: top-k as a per-request tunable; the pages give no
 * formula -- the plainest reading is used:)
 *   logits[t][e] = sum_h x[t][h] * router_w[e][h] + logit_bias[e]   (fp32 sum)
 *   ids[t][j]    = the j-th largest logit of token t, ties to the lower index
 *   softmax: w[t][j] = exp(l_j - l_max) / sum_{i<k} exp(l_i - l_max)
 *            (equal to a softmax over all E renormalised to the selected k)
 *   sigmoid: w[t][j] = s_j / sum_{i<k} s_i,  s = 1 / (1 + exp(-l))
 * x          [T][H]  act_dtype             (unused if logits_in != NULL)
 * router_w   [E][H]  router_dtype          (unused if logits_in != NULL)
 * logit_bias [E]     fp32 or NULL          (unused if logits_in != NULL)
 * logits_in  [T][E]  fp32 or NULL: if set, selection and weights are computed
 *                    from these logits (which already include any bias)
 * logits     [T][E]  fp32 out; required when logits_in is NULL, else may be
 *                    NULL (nothing written)
 * topk_ids   [T][k]  int32 out;  topk_w [T][k] fp32 out.
 * Logits must be finite; ids stay in [0, E) whatever the logits. */
int fw_moe_route(const fw_moe_desc *desc, int32_t T, const void *x, const void *router_w,
                 const float *logit_bias, const float *logits_in, float *logits,
                 int32_t *topk_ids, float *topk_w, void *stream);

/* Token -> expert grouping (the grouped routed-expert kernels' row lists;
 * Flyweight 0.2.0 "Quantization" and "Current limitations").  A stable counting
 * sort of the P = T*k (token, slot) pairs q = t*k + j by expert:
 *   expert_offsets [E+1] int32 out: pairs routed to experts below e;
 *                  expert_offsets[E] = number of valid pairs (P if all ids valid)
 *   sorted_pairs   [P]   int32 out: pair ids, expert-major, ascending q within
 *                  an expert; entries past expert_offsets[E] are -1
 *   inv_pos        [P]   int32 out: sorted_pairs[inv_pos[q]] == q; -1 for a pair
 *                  whose id is out of range (and FW_STATUS_BAD_EXPERT_ID is set)
 * topk_ids [T][k] int32 in.  Up to 2048 pairs the workspace holds the status
 * word only (256 bytes suffice); above that the sort keeps per-1024-pair-chunk
 * expert counts in it and needs fw_moe_workspace_size(desc, T) bytes, else
 * FW_EWORKSPACE.  Bit-exact and unique for valid ids. */
int fw_moe_permute(const fw_moe_desc *desc, int32_t T, const int32_t *topk_ids,
                   int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *inv_pos,
                   void *workspace, size_t ws_bytes, void *stream);

/* Expert FFNs and combine:
 *   for every pair q = (t, j) routed to expert e:
 *     a = SiLU(W_gate[e] x_t) * (W_up[e] x_t),   y_q = W_down[e] a
 *   out[t] = sum_{j<k} topk_w[t][j] * y_{(t,j)}  (slot order)  + shared(x_t)
 * SwiGLU experts: vOOM module layout (the shared block math); the fused
 * gate/up pass that shares each activation load: Flyweight 0.2.0 "Current
 * limitations"; the fixed-order, deterministic combine: vOOM notes (a fused
 * expert path that changed the token stream was rejected).
 * x        [T][H]  act_dtype
 * w_gate, w_up [E][F][H/32] blocks of expert_q;  w_down [E][H][F/32] blocks
 *          (Q4_K, Q6_K: [E][F][H/256] and [E][H][F/256] super-blocks, 144 or
 *          210 bytes each; a Q6_K row is 2-byte aligned when H/256 or F/256
 *          is not a multiple of 8, which the kernels handle.  MXFP4 (MLX
 *          packing, group 32; vOOM notes: expert-only MXFP4, --group-size
 *          32): each projection is its E2M1 codes, [E][F][H/2] bytes
 *          (element j in nibble j % 2 of byte j / 2, low first), followed in
 *          the same buffer by its E8M0 scales, [E][F][H/32] bytes; value =
 *          E2M1(code) * 2^(scale - 127).  Shared: [Fs][H/2] then [Fs][H/32].)
 * ws_gate, ws_up [Fs][H/32], ws_down [H][Fs/32] blocks of shared_q, or NULL
 *          when shared_ffn == 0 (all three required when shared_ffn > 0)
 * topk_w   [T][k] fp32;  expert_offsets, sorted_pairs, inv_pos as produced by
 *          fw_moe_permute (validated on the device: see FW_STATUS_*)
 * out      [T][H] fp32 out (fully overwritten)
 * workspace / ws_bytes: at least fw_moe_workspace_size(desc, T) bytes.
 * Numerics: both families round the activations x and the SwiGLU output h to
 * fp16 and accumulate in fp32.  Each token row is first scaled by a power of
 * two that puts its largest magnitude in [16, 32) (x * 2^e; g and u are
 * scaled back exactly before SwiGLU, h is held at 2^(2e) and the down
 * projection's sums are scaled back exactly), so a finite row of any
 * magnitude uses fp16's normal range like a unit-scale row.  The GEMV family (small T) multiplies the exact
 * weight codes (fp16 holds every Q8_0/Q4_0/Q4_K/Q6_K code, and every E2M1
 * value times 2^-14) by fp16 activations in fp32 dot products and applies
 * each block's scale (Q4_K: each 32-element sub-block's d * scale, and dmin *
 * min times the sub-block's activation sum; Q6_K: each 16-element
 * sub-block's d * scale; MXFP4: 2^(scale - 113), exactly) in fp32; the GEMM
 * family (large T) contracts on fp16 MFMA with weights dequantised to fp16
 * (code times scale, or for Q4_K d * scale * q - dmin * min and for Q6_K
 * d * scale * (q - 32) formed in fp32; one rounding; MXFP4 exactly).  Either way a layer output stays within
 * 2e-3 max-abs and 1e-3 relative L2 of an fp64 evaluation of the same layer
 * for unit-scale inputs like the workloads' (N(0,1) activations, weights of
 * std 0.015-0.02), and each token row within the same relative error at any
 * finite scale.  What fp16 cannot hold is reported, not clamped:
 * FW_STATUS_RANGE is set for a non-finite x, for a scaled h beyond +-65504
 * (very large weights), and, in the GEMM family, for a block scale above
 * 31.98 (Q8_0) or 511.75 (Q4_0) -- 16x the extreme code times the scale must
 * stay within fp16 -- a Q4_K sub-block whose 16 (15 |d scale| + |dmin
 * min|) exceeds 65504, a Q6_K sub-block whose 512 |d scale| does, or an
 * MXFP4 scale above 136 (96 x 2^(scale - 127) beyond fp16; scale 255, NaN
 * by the format, included).  The GEMV family has no weight limit (codes stay
 * exact, scales apply in fp32).
 * With act_quant = FW_ACT_MXFP8 the experts' inputs are MXFP8 (see
 * FW_ACT_MXFP8) and the contraction is the block-scaled MFMA's (E4M3 x E2M1
 * products exact; each 64-product slice summed in the instruction's own
 * accumulation, within ~1e-4 of the slice's sum of |products|); the output
 * then follows an fp64 evaluation of the same MXFP8 layer within 1e-3
 * relative L2, a SwiGLU value on an E4M3 rounding boundary possibly taking
 * the neighbouring code.  FW_STATUS_RANGE is set for non-finite x or h.
 * With act_quant = FW_ACT_INT8 the experts' inputs are int8 blocks (see
 * FW_ACT_INT8): the int32 block sums are exact and each adds (d_x d_w) S in
 * fp32, so the output follows an fp64 evaluation of the same int8 layer
 * within the layer's tolerances, a SwiGLU value within rounding of a code
 * boundary possibly taking the neighbouring code; no fp16 range limits
 * apply.  FW_STATUS_RANGE is set for non-finite x or h.
 * Q4_K and Q6_K (GGUF K-quants, 144- and 210-byte super-blocks of 256
 * elements) need H, F and Fs to be multiples of 256, which every descriptor
 * already is.  MXFP4 requires the routed and shared matrices to be stored
 * as above; a scale of 255 (NaN) gives non-finite outputs in the GEMV.
 * Batch limit: T * k * max(H, F, Fs) < 2^31 (the kernels' row offsets are
 * 32-bit element counts); a larger batch returns FW_EINVAL before anything
 * is enqueued and is to be split by the caller (DeepSeek-shaped layer:
 * up to 37,449 tokens per call).  fw_moe_layer and fw_moe_forward_path apply
 * the same limit. */
int fw_moe_forward(const fw_moe_desc *desc, int32_t T, const void *x, const void *w_gate,
                   const void *w_up, const void *w_down, const void *ws_gate,
                   const void *ws_up, const void *ws_down, const float *topk_w,
                   const int32_t *expert_offsets, const int32_t *sorted_pairs,
                   const int32_t *inv_pos, float *out, void *workspace, size_t ws_bytes,
                   void *stream);

/* The whole layer in one call: fw_moe_route (logits computed, logits_in
 * NULL), fw_moe_permute and fw_moe_forward on the same arguments, with the
 * same results bit for bit (the route of fw_moe_route, the sort of
 * fw_moe_permute, the expert FFNs and combine of fw_moe_forward, as stated
 * above).  When the forward runs the GEMV family (AUTO up to T*k = 2E, or
 * FW_PATH_GEMV) and T*k <= 2048, the top-k, the permutation and the forward's
 * activation staging run as one kernel, so a decode step is five launches
 * instead of seven; otherwise the launches are those of the three calls.
 * Persistent, single-launch decode kernels are listed among the pages' open
 * work (Flyweight 0.2.0 "Current limitations").
 * Arguments: as in the three calls.  logits [T][E] fp32 out, topk_ids
 * [T][k] int32 out, topk_w [T][k] fp32 out, expert_offsets [E+1],
 * sorted_pairs [T*k] and inv_pos [T*k] int32 out are caller-owned device
 * buffers, all required (the layer's intermediate results stay readable);
 * workspace / ws_bytes: at least fw_moe_workspace_size(desc, T) bytes.
 * Every argument is checked before the first launch: an error return means
 * nothing was enqueued.  Asynchronous on `stream`, allocation-free, capturable
 * in a HIP graph. */
int fw_moe_layer(const fw_moe_desc *desc, int32_t T, const void *x, const void *router_w,
                 const float *logit_bias, const void *w_gate, const void *w_up,
                 const void *w_down, const void *ws_gate, const void *ws_up,
                 const void *ws_down, float *logits, int32_t *topk_ids, float *topk_w,
                 int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *inv_pos, float *out,
                 void *workspace, size_t ws_bytes, void *stream);

/* The forward kernel family AUTO picks for T tokens (FW_PATH_GEMV or
 * FW_PATH_GEMM), or a negative error for an invalid descriptor.  AUTO takes
 * the GEMV family while T * k <= 2 * E (at most two routed rows per expert on
 * average) and the grouped GEMM above: the measured crossovers of the
 * hidden-4096 / 64-expert, Qwen3-shaped and DeepSeek-shaped layers lie
 * between 1.5 and 3 rows per expert. */
int fw_moe_forward_path(const fw_moe_desc *desc, int32_t T);

/* Reset the workspace's status word (a fill kernel on `stream`). */
int fw_moe_clear_status(void *workspace, void *stream);

/* Blocking: wait for the device and copy the status word to *host_status.
 * For tests and harnesses, not for the hot path. */
int fw_moe_read_status(const void *workspace, int32_t *host_status);

/* Where a forward call on T tokens keeps its staged expert inputs inside the
 * workspace: byte offsets of the activation staging area (with
 * FW_ACT_MXFP8: x as E4M3 codes [T][H], then the E8M0 scales [T][H/32];
 * with FW_ACT_INT8: int8 codes [T][H], then fp32 scales [T][H/32]) and of the
 * SwiGLU output area (codes [T*k][F] then [T][Fs], then the scales of those
 * rows, one per 32: E8M0 bytes for FW_ACT_MXFP8, fp32 for FW_ACT_INT8).  Host-only; for tests that
 * read those areas back.  FW_OK, or an error for an invalid descriptor / T. */
int fw_moe_workspace_offsets(const fw_moe_desc *desc, int32_t T, size_t *x_stage,
                             size_t *h_stage);

/* Human-readable text of a return code. */
const char *fw_moe_status_string(int status);

/* fw_moe_layer with timing events: the same validation, launches and results
 * as fw_moe_layer, plus HIP events recorded on `stream` around the forward's
 * stages: stage_events[0] before its first kernel and stage_events[s+1]
 * after stage s, s in {0: the fused front end (GEMV batches) or the
 * activation staging, 1: the routed experts' gate/up projection (one
 * launch), 2: the shared expert's gate/up projection (nothing when
 * shared_ffn is 0), 3: down projections, 4: combine}; the logits, top-k and
 * permutation launches that precede stage 0 fall outside.  stage_events: FW_N_STAGE_EVENTS caller-created hipEvent_t
 * handles (required; FW_EINVAL if any is NULL).  For benchmarks and
 * profilers: it keeps no state between calls, so concurrent callers with
 * their own events and workspaces do not interfere. */
enum { FW_N_STAGE_EVENTS = 6 };
int fw_moe_layer_timed(const fw_moe_desc *desc, int32_t T, const void *x,
                       const void *router_w, const float *logit_bias, const void *w_gate,
                       const void *w_up, const void *w_down, const void *ws_gate,
                       const void *ws_up, const void *ws_down, float *logits,
                       int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
                       int32_t *sorted_pairs, int32_t *inv_pos, float *out, void *workspace,
                       size_t ws_bytes, void *const *stage_events, void *stream);

/* fw_moe_layer without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture that must not call
 * hipMalloc, tight serving loops, harnesses that forbid allocation).  The
 * workspace is a static device array of FW_NOALLOC_SCRATCH_BYTES inside the
 * library, one per device, which the library holds from its first use on a
 * device until the process ends; the call itself allocates nothing.
 * Arguments and results: as fw_moe_layer (bit for bit the same outputs), minus
 * workspace / ws_bytes, plus
 *   status  int32 device pointer (4-byte aligned) or NULL: receives the call's
 *           FW_STATUS_* bits when the stream reaches the end of the call.
 * The status word in the array is cleared (a fill kernel) at the start of
 * every call; everything else the kernels need zeroed they clear themselves.
 * Batches whose fw_moe_workspace_size(desc, T) exceeds FW_NOALLOC_SCRATCH_BYTES
 * are refused with FW_EWORKSPACE before anything is enqueued (every decode
 * batch of the workloads here fits; DeepSeek-shaped prefill does not).
 * All calls on one device share its array: calls that overlap on one device
 * (two streams, two threads) race and must be serialised by the caller. */
#define FW_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fw_moe_layer_noalloc(const fw_moe_desc *desc, int32_t T, const void *x,
                         const void *router_w, const float *logit_bias, const void *w_gate,
                         const void *w_up, const void *w_down, const void *ws_gate,
                         const void *ws_up, const void *ws_down, float *logits,
                         int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
                         int32_t *sorted_pairs, int32_t *inv_pos, float *out,
                         int32_t *status, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* FWMOE_H */
