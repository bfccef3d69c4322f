// Microbenchmarks of the two ceilings the layer's kernels are measured
// against: dense fp16 MFMA throughput and HBM streaming-read bandwidth.  Built
// into libfwpeak.so, apart from the layer's library; only the benchmark's peak
// mode loads it.
//
//  - fw_peak_mfma: every wavefront issues chains of independent
//    v_mfma_f32_16x16x32_f16 (or 32x32x16) on register operands, eight
//    accumulators deep so no MFMA waits on the previous one's result; the
//    accumulators are written out at the end so nothing is dead code.
//  - fw_peak_read: a grid-stride read of a buffer with 16-byte loads, four in
//    flight per lane, folded into one XOR per thread that is written out.
//  - fw_peak_copy: the same stride, reading and writing (a copy).
//  - fw_peak_grid_barrier: the price of one grid-wide rendezvous inside a
//    kernel, what a single persistent kernel pays between dependent phases
//    (router logits -> routing, gate/up -> down, down -> combine): every
//    workgroup writes a payload, releases it (optionally behind a full
//    device-scope fence), publishes a per-workgroup flag, polls every flag
//    with relaxed loads and acquires once.  Polls are bounded (they give up
//    after `limit` tries and set *err), so a grid that is not co-resident
//    ends instead of hanging.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

// CH independent accumulator chains per wavefront
template <int CH>
__global__ __launch_bounds__(256) void mfma16_kernel(int iters, float *out) {
    const int lane = threadIdx.x % 64;
    h8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.001f * (lane + i));
        b[i] = (_Float16)(0.002f * (lane - i));
    }
    f4 acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = f4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CH; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int CH>
__global__ __launch_bounds__(256) void mfma32_kernel(int iters, float *out) {
    const int lane = threadIdx.x % 64;
    h8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.001f * (lane + i));
        b[i] = (_Float16)(0.002f * (lane - i));
    }
    f16v acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CH; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_kernel(const uint4 *__restrict__ src, size_t n16,
                                                   uint32_t *__restrict__ out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t x = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride],
                    v3 = src[i + 3 * stride];
        x ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
        x ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = src[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4 *__restrict__ src,
                                                   uint4 *__restrict__ dst, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

// flags: gridDim.x flags 64 bytes apart, zero before the launch
__global__ __launch_bounds__(256) void grid_barrier_kernel(int *flags, float *data, int rounds,
                                                           int limit, int fence,
                                                           int *err) {
    const int G = gridDim.x, wg = blockIdx.x, t = threadIdx.x;
    for (int r = 1; r <= rounds; ++r) {
        data[(size_t)wg * 256 + t] = (float)(r + t);
        if (fence) __threadfence();
        __syncthreads();
        if (t == 0)
            __hip_atomic_store(&flags[wg * 16], r, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        bool ok = true;
        for (int f = t; f < G; f += 256) {
            int n = 0;
            while (__hip_atomic_load(&flags[f * 16], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) < r) {
                if (++n > limit) {
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (!ok) atomicOr(err, 1);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __syncthreads();
        if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
    }
}

}  // namespace

extern "C" {

/* fp16 MFMA throughput: `blocks` workgroups of 256 threads, each wavefront
 * issuing iters * chains MFMAs of 16x16x32 (shape 16; chains 4, 8 or 16) or
 * 32x32x16 (shape 32; chains 2, 4 or 8) -- 16384 or 32768 flops each -- on
 * `chains` independent accumulators.  out: blocks * 256 floats.  Returns a
 * hipError_t. */
int fw_peak_mfma(int shape, int chains, int blocks, int iters, float *out, void *stream) {
    if (blocks < 1 || iters < 1 || !out) return hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)stream;
    if (shape == 16 && chains == 4) mfma16_kernel<4><<<blocks, 256, 0, s>>>(iters, out);
    else if (shape == 16 && chains == 8) mfma16_kernel<8><<<blocks, 256, 0, s>>>(iters, out);
    else if (shape == 16 && chains == 16) mfma16_kernel<16><<<blocks, 256, 0, s>>>(iters, out);
    else if (shape == 32 && chains == 2) mfma32_kernel<2><<<blocks, 256, 0, s>>>(iters, out);
    else if (shape == 32 && chains == 4) mfma32_kernel<4><<<blocks, 256, 0, s>>>(iters, out);
    else if (shape == 32 && chains == 8) mfma32_kernel<8><<<blocks, 256, 0, s>>>(iters, out);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

/* Streaming read of `bytes` (a multiple of 16) from src with `blocks`
 * workgroups of 256 threads; out: blocks * 256 uint32. */
int fw_peak_read(const void *src, size_t bytes, int blocks, uint32_t *out, void *stream) {
    if (!src || !out || bytes % 16 || blocks < 1) return hipErrorInvalidValue;
    read_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const uint4 *)src, bytes / 16, out);
    return hipGetLastError();
}

/* Copy of `bytes` (a multiple of 16) from src to dst with `blocks` workgroups. */
int fw_peak_copy(const void *src, void *dst, size_t bytes, int blocks, void *stream) {
    if (!src || !dst || bytes % 16 || blocks < 1) return hipErrorInvalidValue;
    copy_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>((const uint4 *)src, (uint4 *)dst,
                                                         bytes / 16);
    return hipGetLastError();
}

/* `rounds` grid-wide rendezvous of `blocks` workgroups of 256 threads (see
 * grid_barrier_kernel; fence: a device-scope fence after each round's
 * payload).  flags: blocks * 16 ints, data: blocks * 256 floats, err: one
 * int, all zeroed by the caller; *err != 0 afterwards means a poll gave up
 * (the grid was not co-resident).  blocks must not exceed what the device
 * holds at once. */
int fw_peak_grid_barrier(int blocks, int rounds, int limit, int fence, int *flags, float *data,
                         int *err, void *stream) {
    if (blocks < 1 || rounds < 1 || limit < 1 || !flags || !data || !err)
        return hipErrorInvalidValue;
    grid_barrier_kernel<<<blocks, 256, 0, (hipStream_t)stream>>>(flags, data, rounds, limit,
                                                                 fence, err);
    return hipGetLastError();
}

}  // extern "C"
