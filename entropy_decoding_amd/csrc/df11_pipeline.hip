// Overlapped block pipeline and a BF16 GEMV consumer for gfx950.
//
// "70% Size, 100% Accuracy ... (DFloat11)", abstract: decompression is done
// per transformer block, so that while a model consumes one block's weights
// the next block can already be decompressed.  df11_pipeline_* order that
// overlap with HIP events on two streams and a ring of output buffers;
// df11_gemv_bf16 is a matrix-vector product over the BF16 tensors of one
// block, used as the consumer that reads a decompressed block.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>

#include "df11.h"
#include "df11_launch.h"

struct df11_pipeline {
    hipStream_t decode;
    uint32_t n_slots;
    hipEvent_t ready[DF11_PIPELINE_MAX_SLOTS];     // decompression into the slot is done
    hipEvent_t released[DF11_PIPELINE_MAX_SLOTS];  // the consumer has finished reading it
    bool filled[DF11_PIPELINE_MAX_SLOTS];
    bool was_released[DF11_PIPELINE_MAX_SLOTS];
    uint32_t decode_share;  // workgroups per compute unit for the decode (0: full grid)
};

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kRowsPerWave = 2;

struct GemvArgs {
    const uint16_t *w;
    const float *x;
    float *y;
    uint32_t n;
    uint32_t groups;                                // row groups of kRowsPerWave rows, all tensors
    uint32_t group_start[DF11_GEMV_MAX_TENSORS + 1];
    uint32_t rows[DF11_GEMV_MAX_TENSORS], cols[DF11_GEMV_MAX_TENSORS];
    uint64_t w_off[DF11_GEMV_MAX_TENSORS], x_off[DF11_GEMV_MAX_TENSORS],
        y_off[DF11_GEMV_MAX_TENSORS];
};

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// acc + sum of 8 products, as a sequential chain of fused multiply-adds
__device__ __forceinline__ float dot8(float acc, uint4 w, float4 x0, float4 x1) {
    acc = fmaf(bf16_lo(w.x), x0.x, acc);
    acc = fmaf(bf16_hi(w.x), x0.y, acc);
    acc = fmaf(bf16_lo(w.y), x0.z, acc);
    acc = fmaf(bf16_hi(w.y), x0.w, acc);
    acc = fmaf(bf16_lo(w.z), x1.x, acc);
    acc = fmaf(bf16_hi(w.z), x1.y, acc);
    acc = fmaf(bf16_lo(w.w), x1.z, acc);
    acc = fmaf(bf16_hi(w.w), x1.w, acc);
    return acc;
}

// Sum over the 64 lanes of a wave, in a fixed order (butterfly over lane xor).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Each wave computes kRowsPerWave consecutive rows of one tensor per pass:
// lane l multiplies columns 8l .. 8l + 7 of every 512, so one 16-byte load
// per row per step and the lanes of a wave read 1 KiB of a row contiguously;
// two steps are loaded before either is used, and the x slice is loaded once
// for the wave's rows.  The host orders the tensors longest rows first, so
// the longest dependency chains start first instead of forming a tail.
__global__ __launch_bounds__(kThreads) void df11_gemv(GemvArgs a) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const uint32_t n_waves = gridDim.x * (kThreads / 64);
    for (uint32_t g = wave; g < a.groups; g += n_waves) {
        uint32_t k = 0;
        while (k + 1 < a.n && g >= a.group_start[k + 1]) k++;
        const uint32_t r0 = (g - a.group_start[k]) * kRowsPerWave;
        const uint32_t cols = a.cols[k];
        const uint32_t nr = min(kRowsPerWave, a.rows[k] - r0);
        const uint16_t *w = a.w + a.w_off[k] + uint64_t(r0) * cols;
        const float *x = a.x + a.x_off[k];
        float acc[kRowsPerWave] = {};
        for (uint32_t c = 8 * lane; c < cols; c += 1024) {
            const uint32_t c2 = c + 512;
            const bool two = c2 < cols;
            const float4 x0 = *reinterpret_cast<const float4 *>(x + c);
            const float4 x1 = *reinterpret_cast<const float4 *>(x + c + 4);
            float4 x2 = make_float4(0, 0, 0, 0), x3 = x2;
            if (two) {
                x2 = *reinterpret_cast<const float4 *>(x + c2);
                x3 = *reinterpret_cast<const float4 *>(x + c2 + 4);
            }
            uint4 v[kRowsPerWave][2];
#pragma unroll
            for (uint32_t r = 0; r < kRowsPerWave; r++) {
                if (r < nr) {
                    v[r][0] = *reinterpret_cast<const uint4 *>(w + uint64_t(r) * cols + c);
                    if (two) v[r][1] = *reinterpret_cast<const uint4 *>(w + uint64_t(r) * cols + c2);
                }
            }
#pragma unroll
            for (uint32_t r = 0; r < kRowsPerWave; r++) {
                if (r < nr) {
                    acc[r] = dot8(acc[r], v[r][0], x0, x1);
                    if (two) acc[r] = dot8(acc[r], v[r][1], x2, x3);
                }
            }
        }
#pragma unroll
        for (uint32_t r = 0; r < kRowsPerWave; r++) {
            const float s = wave_sum(acc[r]);
            if (lane == 0 && r < nr) a.y[a.y_off[k] + r0 + r] = s;
        }
    }
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

}  // namespace

extern "C" {

int df11_gemv_bf16(const uint16_t *w, const df11_gemv_tensor *t, uint32_t n_tensors,
                   const float *x, float *y, df11_hip_stream st) {
    if (n_tensors == 0) return DF11_OK;
    if (!t || n_tensors > DF11_GEMV_MAX_TENSORS || !w || !x || !y || !aligned(w, 16) ||
        !aligned(x, 16))
        return DF11_E_INVALID;
    GemvArgs a{};
    a.w = w;
    a.x = x;
    a.y = y;
    a.n = n_tensors;
    // longest rows first (each row is independent, so the order only changes
    // which waves start first)
    uint32_t order[DF11_GEMV_MAX_TENSORS];
    for (uint32_t k = 0; k < n_tensors; k++) order[k] = k;
    std::stable_sort(order, order + n_tensors,
                     [t](uint32_t i, uint32_t j) { return t[i].cols > t[j].cols; });
    uint64_t groups = 0;
    for (uint32_t k = 0; k < n_tensors; k++) {
        const df11_gemv_tensor &d = t[order[k]];
        if (d.cols % 8 || d.w_offset % 8 || d.x_offset % 4) return DF11_E_INVALID;
        a.group_start[k] = uint32_t(groups);
        a.rows[k] = d.rows;
        a.cols[k] = d.cols;
        a.w_off[k] = d.w_offset;
        a.x_off[k] = d.x_offset;
        a.y_off[k] = d.y_offset;
        groups += (uint64_t(d.rows) + kRowsPerWave - 1) / kRowsPerWave;
        if (groups >= (uint64_t(1) << 31)) return DF11_E_INVALID;
    }
    a.group_start[n_tensors] = uint32_t(groups);
    a.groups = uint32_t(groups);
    if (groups == 0) return DF11_OK;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return DF11_E_HIP;
    const uint64_t waves_wanted = groups, per_wg = kThreads / 64;
    const uint64_t grid = std::min<uint64_t>((waves_wanted + per_wg - 1) / per_wg,
                                             uint64_t(std::max(cus, 1)) * 16);
    void *args[] = {&a};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&df11_gemv),
                                         dim3(uint32_t(grid)), dim3(kThreads), args, 0,
                                         static_cast<hipStream_t>(st));
    return e == hipSuccess ? DF11_OK : DF11_E_HIP;
}

int df11_pipeline_create(df11_hip_stream decode_stream, uint32_t n_slots, df11_pipeline **out) {
    if (!out || n_slots < 1 || n_slots > DF11_PIPELINE_MAX_SLOTS) return DF11_E_INVALID;
    *out = nullptr;
    df11_pipeline *p = new (std::nothrow) df11_pipeline{};
    if (!p) return DF11_E_INVALID;
    p->decode = static_cast<hipStream_t>(decode_stream);
    p->n_slots = n_slots;
    for (uint32_t i = 0; i < n_slots; i++) {
        if (hipEventCreateWithFlags(&p->ready[i], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&p->released[i], hipEventDisableTiming) != hipSuccess) {
            df11_pipeline_destroy(p);
            return DF11_E_HIP;
        }
    }
    *out = p;
    return DF11_OK;
}

int df11_pipeline_destroy(df11_pipeline *p) {
    if (!p) return DF11_OK;
    int rc = DF11_OK;
    for (uint32_t i = 0; i < p->n_slots; i++) {
        if (p->ready[i] && hipEventDestroy(p->ready[i]) != hipSuccess) rc = DF11_E_HIP;
        if (p->released[i] && hipEventDestroy(p->released[i]) != hipSuccess) rc = DF11_E_HIP;
    }
    delete p;
    return rc;
}

int df11_pipeline_decompress(df11_pipeline *p, uint32_t slot, const df11_device_stream *s,
                             void *out, int32_t *d_status) {
    if (!p || slot >= p->n_slots) return DF11_E_INVALID;
    // the slot's previous contents must have been released by their consumer
    if (p->was_released[slot] && hipStreamWaitEvent(p->decode, p->released[slot], 0) != hipSuccess)
        return DF11_E_HIP;
    const int rc = df11_detail::decompress_block_capped(s, out, d_status, p->decode,
                                                        p->decode_share);
    if (rc != DF11_OK) return rc;
    if (hipEventRecord(p->ready[slot], p->decode) != hipSuccess) return DF11_E_HIP;
    p->filled[slot] = true;
    return DF11_OK;
}

int df11_pipeline_set_decode_share(df11_pipeline *p, uint32_t workgroups_per_cu) {
    if (!p || workgroups_per_cu > 64) return DF11_E_INVALID;
    p->decode_share = workgroups_per_cu;
    return DF11_OK;
}

int df11_pipeline_acquire(df11_pipeline *p, uint32_t slot, df11_hip_stream consumer) {
    if (!p || slot >= p->n_slots || !p->filled[slot]) return DF11_E_INVALID;
    return hipStreamWaitEvent(static_cast<hipStream_t>(consumer), p->ready[slot], 0) == hipSuccess
               ? DF11_OK
               : DF11_E_HIP;
}

int df11_pipeline_release(df11_pipeline *p, uint32_t slot, df11_hip_stream consumer) {
    if (!p || slot >= p->n_slots || !p->filled[slot]) return DF11_E_INVALID;
    if (hipEventRecord(p->released[slot], static_cast<hipStream_t>(consumer)) != hipSuccess)
        return DF11_E_HIP;
    p->was_released[slot] = true;
    return DF11_OK;
}

}  // extern "C"
