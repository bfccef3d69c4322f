// The C ABI (declared in include/fwmoe.h): argument validation, workspace
// layout, kernel-family choice and the launch sequence of each entry point.
// Everything here runs on the host and enqueues asynchronously; nothing is
// allocated and nothing waits, except fw_moe_read_status.
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "common.h"

// Workspace of fw_moe_layer_noalloc, for callers that cannot allocate: one
// array per device, held from the library's first use on that device until
// the process ends.  Host code never names it in a launch or copy: its device
// address comes from hipGetSymbolAddress, once per device (noalloc_scratch).
constexpr size_t kNoAllocScratchBytes = FW_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace fw {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(const fw_moe_desc &d, int T) {
    WsLayout L{};
    const size_t H = d.hidden, F = d.ffn, Fs = d.shared_ffn, E = d.n_experts;
    const size_t P = (size_t)T * d.top_k;
    size_t off = sizeof(WsHeader);
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    // row tiles of either family: GEMM tiles of 128 or 160 rows, GEMV chunks
    // of kGemvTokens rows (the larger count)
    L.max_tiles = (int)((P + kGemvTokens - 1) / kGemvTokens + E);
    L.active = take((E + 1) * sizeof(int4));
    L.tiles = take((size_t)L.max_tiles * sizeof(int4));
    L.x16 = take((size_t)T * H * 2);
    L.h = take((P * F + (size_t)T * Fs) * 2);
    L.y = take((P + (Fs ? (size_t)T : 0)) * H * 4);
    L.split_cnt = take((size_t)kSplitTiles * 4);
    L.split_part = take((size_t)kSplitTiles * kSplitSlicesMax * 2 * kGemvTokens * kWave * 4);
    L.xe = take((size_t)T * 4);
    L.he = take((P + (size_t)T) * 4);
    L.xsum = take((size_t)T * (H / 32) * 4);
    L.hsum = take((P * (F / 32) + (size_t)T * (Fs / 32)) * 4);
    L.perm = take(E * (size_t)(perm_blocks((long long)P) + 1) * 4);
    L.total = off;
    return L;
}

}  // namespace fw

using namespace fw;

namespace {

bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }
bool al256(const void *p) { return ((uintptr_t)p & 255) == 0; }

int check_desc(const fw_moe_desc *d) {
    if (!d) return FW_EINVAL;
    if (d->hidden < 256 || d->hidden > 16384 || d->hidden % 256) return FW_EINVAL;
    if (d->n_experts < 1 || d->n_experts > kMaxExperts) return FW_EINVAL;
    if (d->top_k < 1 || d->top_k > std::min(d->n_experts, kMaxTopK)) return FW_EINVAL;
    if (d->ffn < 256 || d->ffn > 16384 || d->ffn % 256) return FW_EINVAL;
    if (d->shared_ffn < 0 || d->shared_ffn > 16384 || d->shared_ffn % 256) return FW_EINVAL;
    if (d->act_dtype != FW_F32 && d->act_dtype != FW_BF16) return FW_EINVAL;
    if (d->router_dtype != FW_F32 && d->router_dtype != FW_BF16) return FW_EINVAL;
    if (d->expert_q < FW_Q8_0 || d->expert_q > FW_MXFP4) return FW_EINVAL;
    if (d->shared_q < FW_Q8_0 || d->shared_q > FW_MXFP4) return FW_EINVAL;
    if (d->score != FW_SOFTMAX_RENORM && d->score != FW_SIGMOID_RENORM) return FW_EINVAL;
    if (d->path < FW_PATH_AUTO || d->path > FW_PATH_GEMM) return FW_EINVAL;
    if (d->act_quant < FW_ACT_NONE || d->act_quant > FW_ACT_INT8) return FW_EINVAL;
    if (d->router_dtype != d->act_dtype) return FW_EUNSUPPORTED;
    if (d->act_quant == FW_ACT_MXFP8 &&
        (d->expert_q != FW_MXFP4 || (d->shared_ffn > 0 && d->shared_q != FW_MXFP4) ||
         d->path == FW_PATH_GEMV))
        return FW_EUNSUPPORTED;
    auto mmq = [](int q) { return q == FW_Q8_0 || q == FW_Q4_0; };
    if (d->act_quant == FW_ACT_INT8 &&
        (!mmq(d->expert_q) || (d->shared_ffn > 0 && !mmq(d->shared_q)) ||
         d->path == FW_PATH_GEMV))
        return FW_EUNSUPPORTED;
    return FW_OK;
}

int check_T(const fw_moe_desc *d, int32_t T) {
    if (T < 0 || T > (1 << 20) || (int64_t)T * d->top_k > (1 << 24)) return FW_EINVAL;
    return FW_OK;
}

// The forward kernels index activation and intermediate rows with 32-bit
// element offsets (row * K): batches whose T * k * max(H, F, Fs) reaches 2^31
// are refused; the caller splits them.
int check_forward_T(const fw_moe_desc *d, int32_t T) {
    const int64_t widest = std::max({d->hidden, d->ffn, d->shared_ffn});
    if ((int64_t)T * d->top_k * widest >= (int64_t)1 << 31) return FW_EINVAL;
    return FW_OK;
}

int resolve_path(const fw_moe_desc *d, int32_t T) {
    if (d->path != FW_PATH_AUTO) return d->path;
    // block-scaled MFMA / int8 MFMA: the grouped GEMM family only
    if (d->act_quant != FW_ACT_NONE) return FW_PATH_GEMM;
    const int64_t pairs = (int64_t)T * d->top_k;
    return pairs <= (int64_t)kGemvMaxRowsPerExpert * d->n_experts ? FW_PATH_GEMV : FW_PATH_GEMM;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FW_OK : FW_EHIP; }

// Checks fw_moe_forward's arguments (desc and T already checked, T > 0) and
// fills the launch arguments.
int forward_args(const fw_moe_desc *desc, int32_t T, const void *x, const void *w_gate,
                 const void *w_up, const void *w_down, const void *ws_gate, const void *ws_up,
                 const void *ws_down, const float *topk_w, const int32_t *expert_offsets,
                 const int32_t *sorted_pairs, const int32_t *inv_pos, float *out,
                 void *workspace, size_t ws_bytes, FwdArgs *out_args) {
    if (check_forward_T(desc, T) != FW_OK) return FW_EINVAL;
    const bool shared = desc->shared_ffn > 0;
    if (!x || !w_gate || !w_up || !w_down || !topk_w || !expert_offsets || !sorted_pairs ||
        !inv_pos || !out || !workspace)
        return FW_EINVAL;
    if (shared && (!ws_gate || !ws_up || !ws_down)) return FW_EINVAL;
    const void *ptrs[] = {x, w_gate, w_up, w_down, topk_w, expert_offsets, sorted_pairs,
                          inv_pos, out};
    for (const void *p : ptrs)
        if (!al16(p)) return FW_EALIGN;
    if (shared && (!al16(ws_gate) || !al16(ws_up) || !al16(ws_down))) return FW_EALIGN;
    if (!al256(workspace)) return FW_EALIGN;
    FwdArgs &a = *out_args;
    a.d = *desc;
    a.T = T;
    a.P = T * desc->top_k;
    a.path = resolve_path(desc, T);
    a.L = ws_layout(*desc, T);
    if (ws_bytes < a.L.total) return FW_EWORKSPACE;
    a.x = x;
    a.wg = (const uint8_t *)w_gate;
    a.wu = (const uint8_t *)w_up;
    a.wd = (const uint8_t *)w_down;
    a.sg = shared ? (const uint8_t *)ws_gate : nullptr;
    a.su = shared ? (const uint8_t *)ws_up : nullptr;
    a.sd = shared ? (const uint8_t *)ws_down : nullptr;
    a.topk_w = topk_w;
    a.offsets = expert_offsets;
    a.sorted = sorted_pairs;
    a.inv = inv_pos;
    a.out = out;
    a.ws = (char *)workspace;
    return FW_OK;
}

// The routing buffers the fused decode front end writes.
struct FrontArgs {
    const float *logits;
    int32_t *ids;
    float *w;
    int32_t *offsets, *sorted, *inv;
};

// The forward's launches: staging (or, with `front`, the fused top-k +
// permutation + staging kernel), gate/up, down, combine; with `ev`
// (FW_N_STAGE_EVENTS events) an event before the first and after each, the
// routed experts' gate/up launch timed apart from the shared expert's.
int enqueue_forward(const FwdArgs &a, const FrontArgs *front, const hipEvent_t *ev,
                    hipStream_t s) {
    int rc;
    if (ev) (void)hipEventRecord(ev[0], s);
    rc = hip_status(front ? launch_decode_front(a, front->logits, front->ids, front->w,
                                                front->offsets, front->sorted, front->inv, s)
                          : launch_prepare(a, s));
    if (rc != FW_OK) return rc;
    if (ev) (void)hipEventRecord(ev[1], s);
    const bool gemm = a.path == FW_PATH_GEMM;
    const hipEvent_t routed_done = ev ? ev[2] : nullptr;
    rc = hip_status(gemm ? launch_gemm_gate_up(a, routed_done, s)
                         : launch_gemv_gate_up(a, routed_done, s));
    if (rc != FW_OK) return rc;
    if (ev) (void)hipEventRecord(ev[3], s);
    rc = hip_status(gemm ? launch_gemm_down(a, s) : launch_gemv_down(a, s));
    if (rc != FW_OK) return rc;
    if (ev) (void)hipEventRecord(ev[4], s);
    if ((rc = hip_status(launch_combine(a, s))) != FW_OK) return rc;
    if (ev) (void)hipEventRecord(ev[5], s);
    return FW_OK;
}

// The launches of fw_moe_layer after validation.
int layer_launches(const FwdArgs &a, const fw_moe_desc *desc, int32_t T, const void *x,
                   const void *router_w, const float *logit_bias, float *logits,
                   int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
                   int32_t *sorted_pairs, int32_t *inv_pos, const hipEvent_t *ev, hipStream_t s) {
    int rc;
    if ((rc = hip_status(launch_logits(*desc, T, x, router_w, logit_bias, logits, s))) != FW_OK)
        return rc;
    if (decode_front_fits(*desc, T, a.path)) {
        FrontArgs f{logits, topk_ids, topk_w, expert_offsets, sorted_pairs, inv_pos};
        return enqueue_forward(a, &f, ev, s);
    }
    if ((rc = hip_status(launch_topk(*desc, T, logits, topk_ids, topk_w, s))) != FW_OK) return rc;
    const long long P = (long long)T * desc->top_k;
    int32_t *perm = P > kPermOneBlockMaxP ? (int32_t *)(a.ws + a.L.perm) : nullptr;
    rc = hip_status(launch_permute(*desc, T, topk_ids, expert_offsets, sorted_pairs, inv_pos,
                                   (WsHeader *)a.ws, perm, s));
    if (rc != FW_OK) return rc;
    return enqueue_forward(a, nullptr, ev, s);
}

// fw_moe_layer: every argument of the three stages is checked before anything
// is enqueued; `ev` as in enqueue_forward.  With `fresh_status` the status
// word is cleared first (a fill kernel) and, when `status_out` is set, copied
// there after the last stage.
int layer_impl(const fw_moe_desc *desc, int32_t T, const void *x, const void *router_w,
               const float *logit_bias, const void *w_gate, const void *w_up,
               const void *w_down, const void *ws_gate, const void *ws_up, const void *ws_down,
               float *logits, int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
               int32_t *sorted_pairs, int32_t *inv_pos, float *out, void *workspace,
               size_t ws_bytes, const hipEvent_t *ev, hipStream_t s, bool fresh_status = false,
               int32_t *status_out = nullptr) {
    int rc = check_desc(desc);
    if (rc != FW_OK) return rc;
    if ((rc = check_T(desc, T)) != FW_OK) return rc;
    if (T == 0) return FW_OK;
    if (!router_w || !logits || !topk_ids || !topk_w || !expert_offsets) return FW_EINVAL;
    if (!al16(router_w) || !al16(logits) || !al16(topk_ids) || (logit_bias && !al16(logit_bias)))
        return FW_EALIGN;
    FwdArgs a;
    rc = forward_args(desc, T, x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, topk_w,
                      expert_offsets, sorted_pairs, inv_pos, out, workspace, ws_bytes, &a);
    if (rc != FW_OK) return rc;
    if (fresh_status &&
        (rc = hip_status(launch_clear_status((WsHeader *)workspace, s))) != FW_OK)
        return rc;
    rc = layer_launches(a, desc, T, x, router_w, logit_bias, logits, topk_ids, topk_w,
                        expert_offsets, sorted_pairs, inv_pos, ev, s);
    if (rc != FW_OK || !status_out) return rc;
    return hip_status(launch_copy_status((const WsHeader *)workspace, status_out, s));
}

// The device address of `scratch` on the current device, looked up once per
// device with that device current (nullptr if the lookup failed).
void *noalloc_scratch() {
    static std::once_flag once[kMaxDevices];
    static void *ptr[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(once[dev], [dev] {
        void *p = nullptr;
        ptr[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
    });
    return ptr[dev];
}

}  // namespace

extern "C" {

const char *fw_moe_version(void) { return "fwmoe 0.1.0 gfx950"; }

int fw_moe_validate(const fw_moe_desc *desc) { return check_desc(desc); }

size_t fw_moe_workspace_size(const fw_moe_desc *desc, int32_t max_T) {
    if (check_desc(desc) != FW_OK || check_T(desc, max_T) != FW_OK) return 0;
    return ws_layout(*desc, max_T).total;
}

int fw_moe_forward_path(const fw_moe_desc *desc, int32_t T) {
    int rc = check_desc(desc);
    if (rc != FW_OK) return rc;
    if ((rc = check_T(desc, T)) != FW_OK) return rc;
    if ((rc = check_forward_T(desc, T)) != FW_OK) return rc;
    return resolve_path(desc, T);
}

int fw_moe_workspace_offsets(const fw_moe_desc *desc, int32_t T, size_t *x_stage,
                             size_t *h_stage) {
    int rc = check_desc(desc);
    if (rc != FW_OK) return rc;
    if ((rc = check_T(desc, T)) != FW_OK) return rc;
    if (!x_stage || !h_stage) return FW_EINVAL;
    const WsLayout L = ws_layout(*desc, T);
    *x_stage = L.x16;
    *h_stage = L.h;
    return FW_OK;
}

int fw_moe_route(const fw_moe_desc *desc, int32_t T, const void *x, const void *router_w,
                 const float *logit_bias, const float *logits_in, float *logits,
                 int32_t *topk_ids, float *topk_w, void *stream) {
    int rc = check_desc(desc);
    if (rc != FW_OK) return rc;
    if ((rc = check_T(desc, T)) != FW_OK) return rc;
    if (T == 0) return FW_OK;
    if (!topk_ids || !topk_w) return FW_EINVAL;
    if (!al16(topk_ids) || !al16(topk_w)) return FW_EALIGN;
    const float *scores = logits_in;
    if (!logits_in) {
        if (!x || !router_w || !logits) return FW_EINVAL;
        if (!al16(x) || !al16(router_w) || !al16(logits) || (logit_bias && !al16(logit_bias)))
            return FW_EALIGN;
        scores = logits;
    } else if (!al16(logits_in)) {
        return FW_EALIGN;
    }
    hipStream_t s = (hipStream_t)stream;
    if (!logits_in) {
        rc = hip_status(launch_logits(*desc, T, x, router_w, logit_bias, logits, s));
        if (rc != FW_OK) return rc;
    }
    return hip_status(launch_topk(*desc, T, scores, topk_ids, topk_w, s));
}

int fw_moe_permute(const fw_moe_desc *desc, int32_t T, const int32_t *topk_ids,
                   int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *inv_pos,
                   void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_desc(desc);
    if (rc != FW_OK) return rc;
    if ((rc = check_T(desc, T)) != FW_OK) return rc;
    if (!expert_offsets || !workspace) return FW_EINVAL;
    if (T > 0 && (!topk_ids || !sorted_pairs || !inv_pos)) return FW_EINVAL;
    if (!al16(expert_offsets) || !al256(workspace) || (T > 0 && (!al16(topk_ids) ||
        !al16(sorted_pairs) || !al16(inv_pos))))
        return FW_EALIGN;
    if (ws_bytes < sizeof(WsHeader)) return FW_EWORKSPACE;
    const long long P = (long long)T * desc->top_k;
    int32_t *perm = nullptr;
    if (P > kPermOneBlockMaxP) {
        const WsLayout L = ws_layout(*desc, T);
        if (ws_bytes < L.total) return FW_EWORKSPACE;
        perm = (int32_t *)((char *)workspace + L.perm);
    }
    return hip_status(launch_permute(*desc, T, topk_ids, expert_offsets, sorted_pairs, inv_pos,
                                     (WsHeader *)workspace, perm, (hipStream_t)stream));
}

int fw_moe_forward(const fw_moe_desc *desc, int32_t T, const void *x, const void *w_gate,
                   const void *w_up, const void *w_down, const void *ws_gate,
                   const void *ws_up, const void *ws_down, const float *topk_w,
                   const int32_t *expert_offsets, const int32_t *sorted_pairs,
                   const int32_t *inv_pos, float *out, void *workspace, size_t ws_bytes,
                   void *stream) {
    int rc = check_desc(desc);
    if (rc != FW_OK) return rc;
    if ((rc = check_T(desc, T)) != FW_OK) return rc;
    if (T == 0) return FW_OK;
    FwdArgs a;
    rc = forward_args(desc, T, x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, topk_w,
                      expert_offsets, sorted_pairs, inv_pos, out, workspace, ws_bytes, &a);
    if (rc != FW_OK) return rc;
    return enqueue_forward(a, nullptr, nullptr, (hipStream_t)stream);
}

int fw_moe_layer(const fw_moe_desc *desc, int32_t T, const void *x, const void *router_w,
                 const float *logit_bias, const void *w_gate, const void *w_up,
                 const void *w_down, const void *ws_gate, const void *ws_up,
                 const void *ws_down, float *logits, int32_t *topk_ids, float *topk_w,
                 int32_t *expert_offsets, int32_t *sorted_pairs, int32_t *inv_pos, float *out,
                 void *workspace, size_t ws_bytes, void *stream) {
    return layer_impl(desc, T, x, router_w, logit_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                      ws_down, logits, topk_ids, topk_w, expert_offsets, sorted_pairs, inv_pos,
                      out, workspace, ws_bytes, nullptr, (hipStream_t)stream);
}

int fw_moe_layer_timed(const fw_moe_desc *desc, int32_t T, const void *x,
                       const void *router_w, const float *logit_bias, const void *w_gate,
                       const void *w_up, const void *w_down, const void *ws_gate,
                       const void *ws_up, const void *ws_down, float *logits,
                       int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
                       int32_t *sorted_pairs, int32_t *inv_pos, float *out, void *workspace,
                       size_t ws_bytes, void *const *stage_events, void *stream) {
    if (!stage_events) return FW_EINVAL;
    for (int i = 0; i < FW_N_STAGE_EVENTS; ++i)
        if (!stage_events[i]) return FW_EINVAL;
    return layer_impl(desc, T, x, router_w, logit_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                      ws_down, logits, topk_ids, topk_w, expert_offsets, sorted_pairs, inv_pos,
                      out, workspace, ws_bytes, (const hipEvent_t *)stage_events,
                      (hipStream_t)stream);
}

int fw_moe_layer_noalloc(const fw_moe_desc *desc, int32_t T, const void *x,
                         const void *router_w, const float *logit_bias, const void *w_gate,
                         const void *w_up, const void *w_down, const void *ws_gate,
                         const void *ws_up, const void *ws_down, float *logits,
                         int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
                         int32_t *sorted_pairs, int32_t *inv_pos, float *out,
                         int32_t *status, void *stream) {
    int rc = check_desc(desc);
    if (rc != FW_OK) return rc;
    if ((rc = check_T(desc, T)) != FW_OK) return rc;
    if (T == 0) return FW_OK;
    if (ws_layout(*desc, T).total > kNoAllocScratchBytes) return FW_EWORKSPACE;
    if (status && ((uintptr_t)status & 3)) return FW_EALIGN;
    void *ws = noalloc_scratch();
    if (!ws) return FW_EHIP;
    return layer_impl(desc, T, x, router_w, logit_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                      ws_down, logits, topk_ids, topk_w, expert_offsets, sorted_pairs, inv_pos,
                      out, ws, kNoAllocScratchBytes, nullptr, (hipStream_t)stream, true, status);
}

int fw_moe_clear_status(void *workspace, void *stream) {
    if (!workspace) return FW_EINVAL;
    if (!al256(workspace)) return FW_EALIGN;
    return hip_status(launch_clear_status((WsHeader *)workspace, (hipStream_t)stream));
}

int fw_moe_read_status(const void *workspace, int32_t *host_status) {
    if (!workspace || !host_status) return FW_EINVAL;
    if (hipDeviceSynchronize() != hipSuccess) return FW_EHIP;
    return hip_status(hipMemcpy(host_status, workspace, sizeof(int32_t), hipMemcpyDeviceToHost));
}

const char *fw_moe_status_string(int status) {
    switch (status) {
        case FW_OK: return "ok";
        case FW_EINVAL: return "invalid argument";
        case FW_EUNSUPPORTED: return "unsupported combination";
        case FW_EWORKSPACE: return "workspace missing or too small";
        case FW_EALIGN: return "misaligned pointer";
        case FW_EHIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

}  // extern "C"
