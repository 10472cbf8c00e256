// Measurement probe for the benchmark (not part of the libgdn ABI): the
// state stream of a multi-slot decode step with nothing else.  For each of
// n entries, slot ids[i]'s fp32 state tiles are read once and written once
// in place (times a runtime scale, 1.0 in the benchmark), with the decode
// kernel's access pattern: each 128-wide row split over 16 lanes of two
// 16-byte segments, 16 rows per pass, every load of a thread issued before
// its first store, non-temporal stores; one or two value-head tiles per
// workgroup and default or non-temporal loads (four variants).  The best
// variant's rate is the ceiling the decode step's state traffic can reach
// with these slot ids, measured on the same box.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kD = 128;
constexpr int kHeadThreads = 256;
constexpr int kLanesPerRow = kD / 8;
constexpr int kRowsPerPass = kHeadThreads / kLanesPerRow;
constexpr int kPasses = kD / kRowsPerPass;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// HEADS value-head tiles per workgroup (kHeadThreads threads each); loads
// with cache policy LOADPOL (0 default, 2 non-temporal), stores non-temporal.
template <int HEADS, int LOADPOL>
__global__ __launch_bounds__(HEADS * kHeadThreads) void stream_tiles_kernel(
    float* __restrict__ state, int heads_per_slot, const int32_t* __restrict__ ids, float scale) {
    const int blk = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
    const int slot = ids[i];
    if (slot < 0) return;
    const int sub = __builtin_amdgcn_readfirstlane(tid / kHeadThreads);
    const int ht = tid % kHeadThreads;
    const int lr = ht % kLanesPerRow, row0 = ht / kLanesPerRow;
    const int voff = (row0 * kD + 4 * lr) * (int)sizeof(float);
    constexpr int kSeg1 = kD / 2 * (int)sizeof(float);
    constexpr int kPass = kRowsPerPass * kD * (int)sizeof(float);
    float* tile = state + ((int64_t)slot * heads_per_slot + HEADS * blk + sub) * kD * kD;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(tile, 0, kD * kD * (int)sizeof(float), 0x00020000);
    f32x4 x[kPasses][2];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        x[p][0] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, p * kPass, LOADPOL);
        x[p][1] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + kSeg1, p * kPass, LOADPOL);
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        __builtin_amdgcn_raw_buffer_store_b128(x[p][0] * scale, rs, voff, p * kPass, 2);
        __builtin_amdgcn_raw_buffer_store_b128(x[p][1] * scale, rs, voff + kSeg1, p * kPass, 2);
    }
}

template <int HEADS, int LOADPOL>
hipError_t launch(float* state, int heads_per_slot, const int32_t* ids, int n, float scale,
                  hipStream_t stream) {
    hipLaunchKernelGGL((stream_tiles_kernel<HEADS, LOADPOL>), dim3(heads_per_slot / HEADS, n),
                       dim3(HEADS * kHeadThreads), 0, stream, state, heads_per_slot, ids, scale);
    return hipGetLastError();
}

}  // namespace

// state: fp32 [n_slots][heads_per_slot][128][128] (device); ids: int32 [n]
// (device, distinct, < n_slots); heads_per_slot even.  variant: bit 0 ->
// non-temporal loads (else default policy), bit 1 -> one value-head tile per
// 256-thread workgroup (else two per 512-thread workgroup, as the decode
// kernel).  Returns a hipError_t value (0 on success).
extern "C" int gdn_probe_stream_tiles(float* state, int heads_per_slot, const int32_t* ids, int n,
                                      float scale, int variant, void* stream) {
    if (!state || !ids || n <= 0 || n > 65535 || heads_per_slot <= 0 || heads_per_slot % 2 ||
        variant < 0 || variant > 3)
        return (int)hipErrorInvalidValue;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (variant) {
        case 0: return (int)launch<2, 0>(state, heads_per_slot, ids, n, scale, s);
        case 1: return (int)launch<2, 2>(state, heads_per_slot, ids, n, scale, s);
        case 2: return (int)launch<1, 0>(state, heads_per_slot, ids, n, scale, s);
        default: return (int)launch<1, 2>(state, heads_per_slot, ids, n, scale, s);
    }
}
