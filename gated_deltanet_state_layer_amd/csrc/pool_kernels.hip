// Pool bookkeeping kernels: zero fill (pool creation, error-word clear) and
// slot reset.  Both write with 16-byte vector stores; no memset nodes are
// used, so the calls can be recorded into a HIP graph.
#include "gdn_common.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void fill_zero_kernel(float4* p, size_t n16) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t j = (size_t)blockIdx.x * kThreads + threadIdx.x; j < n16; j += stride)
        p[j] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// A reused request slot starts from zero: clear its state tiles and conv
// windows and empty its verify rings for every layer ("Project: adding the hybrid model Qwen3.5",
// "What to do", row "State").  grid = (blocks per slot, n entries).
__global__ __launch_bounds__(kThreads) void slot_reset_kernel(PoolView P, const int32_t* slot_ids,
                                                             size_t state16_per_slot,
                                                             size_t window16_per_slot) {
    const int slot = slot_ids[blockIdx.y];
    if (slot < 0) return;
    if (slot >= P.n_slots) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(P.err, kErrSlotRange);
        return;
    }
    float4* st = reinterpret_cast<float4*>(P.state) + (size_t)slot * state16_per_slot;
    float4* wn = reinterpret_cast<float4*>(P.window) + (size_t)slot * window16_per_slot;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t j = (size_t)blockIdx.x * kThreads + threadIdx.x; j < state16_per_slot; j += stride) st[j] = z;
    for (size_t j = (size_t)blockIdx.x * kThreads + threadIdx.x; j < window16_per_slot; j += stride) wn[j] = z;
    // an empty verify ring (its records need no clearing)
    if (P.ring_len > 0 && blockIdx.x == 0)
        for (int l = threadIdx.x; l < P.n_layers; l += kThreads) P.ring_cnt[(int64_t)slot * P.n_layers + l] = 0;
}

// Copy the state tiles, conv windows and verify rings of every layer of slot
// src_ids[i] to slot dst_ids[i] (a state "saved and copied whole": "Project: adding the
// hybrid model Qwen3.5", prefix-cache notes).  grid = (blocks per slot, n).
__global__ __launch_bounds__(kThreads) void slot_copy_kernel(PoolView P, const int32_t* src_ids,
                                                            const int32_t* dst_ids,
                                                            size_t state16_per_slot,
                                                            size_t window16_per_slot) {
    const int src = src_ids[blockIdx.y], dst = dst_ids[blockIdx.y];
    if (src < 0 || dst < 0) return;
    if (src >= P.n_slots || dst >= P.n_slots) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(P.err, kErrSlotRange);
        return;
    }
    const float4* ss = reinterpret_cast<const float4*>(P.state) + (size_t)src * state16_per_slot;
    float4* sd = reinterpret_cast<float4*>(P.state) + (size_t)dst * state16_per_slot;
    const float4* ws = reinterpret_cast<const float4*>(P.window) + (size_t)src * window16_per_slot;
    float4* wd = reinterpret_cast<float4*>(P.window) + (size_t)dst * window16_per_slot;
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t j = (size_t)blockIdx.x * kThreads + threadIdx.x; j < state16_per_slot; j += stride) sd[j] = ss[j];
    for (size_t j = (size_t)blockIdx.x * kThreads + threadIdx.x; j < window16_per_slot; j += stride) wd[j] = ws[j];
    if (P.ring_len > 0) {   // the verify ring: counts and records of every layer
        const size_t ring16 = (size_t)P.n_layers * P.ring_stride / 4;
        const float4* rs = reinterpret_cast<const float4*>(P.ring) + (size_t)src * ring16;
        float4* rd = reinterpret_cast<float4*>(P.ring) + (size_t)dst * ring16;
        for (size_t j = (size_t)blockIdx.x * kThreads + threadIdx.x; j < ring16; j += stride) rd[j] = rs[j];
        if (blockIdx.x == 0)
            for (int l = threadIdx.x; l < P.n_layers; l += kThreads)
                P.ring_cnt[(int64_t)dst * P.n_layers + l] = P.ring_cnt[(int64_t)src * P.n_layers + l];
    }
}

}  // namespace

hipError_t launch_slot_copy(const gdn_pool* pool, int32_t n, const int32_t* src_ids,
                            const int32_t* dst_ids, hipStream_t stream) {
    const PoolView& P = pool->view;
    const size_t state16 = (size_t)P.n_layers * P.h_v * P.d * P.d / 4;
    const size_t win16 = (size_t)P.n_layers * (P.conv_k - 1) * P.c_conv * pool->io_size / 16;
    size_t blocks = (state16 + kThreads * 4 - 1) / (kThreads * 4);
    blocks = blocks < 1 ? 1 : (blocks > 256 ? 256 : blocks);
    hipLaunchKernelGGL(slot_copy_kernel, dim3((unsigned)blocks, n), dim3(kThreads), 0, stream, P,
                       src_ids, dst_ids, state16, win16);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;  // callers pass multiples of 16 bytes
    if (n16 == 0) return hipSuccess;
    size_t blocks = (n16 + kThreads - 1) / kThreads;
    blocks = blocks > 4096 ? 4096 : blocks;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<float4*>(ptr), n16);
    return hipGetLastError();
}

hipError_t launch_slot_reset(const gdn_pool* pool, int32_t n, const int32_t* slot_ids,
                             hipStream_t stream) {
    const PoolView& P = pool->view;
    const size_t state16 = (size_t)P.n_layers * P.h_v * P.d * P.d / 4;
    const size_t win_bytes = (size_t)P.n_layers * (P.conv_k - 1) * P.c_conv * pool->io_size;
    const size_t win16 = win_bytes / 16;  // c_conv is a multiple of 32, so this is exact
    size_t blocks = (state16 + kThreads * 4 - 1) / (kThreads * 4);
    blocks = blocks < 1 ? 1 : (blocks > 256 ? 256 : blocks);
    hipLaunchKernelGGL(slot_reset_kernel, dim3((unsigned)blocks, n), dim3(kThreads), 0, stream, P,
                       slot_ids, state16, win16);
    return hipGetLastError();
}

}  // namespace gdn
