// Shared device helpers and the internal launcher interface of libgdn.
// gfx950 (CDNA4) only: wave64, DPP cross-lane moves, bf16 storage.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gdn.h"

namespace gdn {

constexpr int kMaxConvK = 8;
constexpr int kMaxVerifyTokens = 8;

// Sticky error bits written to the pool's meta word.
constexpr int kErrSlotRange = 1;
constexpr int kErrSeqlens = 2;

// ----------------------------------------------------------------- bf16 / io

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Activation element access for the two io dtypes.
template <typename T> struct Io;
template <> struct Io<float> {
    __device__ static __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    __device__ static __forceinline__ void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct Io<uint16_t> {
    __device__ static __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ static __forceinline__ void store(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
};

// ----------------------------------------------------------- cross-lane sums

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W lanes (W = 2, 4, 8 or 16); every lane of the
// group receives the sum.  Uses DPP inside 16-lane rows: quad swaps, then the
// half-row and row mirrors (after the quad steps every quad holds its own sum,
// so any pairing of quads completes the reduction).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group width");
    x += dpp_mov<0xB1>(x);                      // quad_perm [1,0,3,2]
    if constexpr (W >= 4) x += dpp_mov<0x4E>(x); // quad_perm [2,3,0,1]
    if constexpr (W >= 8) x += dpp_mov<0x141>(x); // row_half_mirror
    if constexpr (W >= 16) x += dpp_mov<0x140>(x); // row_mirror
    return x;
}

// Full 64-lane sum, result in every lane.
__device__ __forceinline__ float wave_sum(float x) {
    x = group_sum<16>(x);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ------------------------------------------------------------ pool (device)

struct PoolView {
    float* state;         // [n_slots][n_layers][h_v][d_v][d_k]
    void* window;         // [n_slots][n_layers][conv_k-1][C_conv] io dtype
    int32_t* err;         // sticky error word
    int32_t* ctr;         // [n_slots][n_layers][h_k] arrival counters of the row-split decode
                          // and the ring commit (0 between calls)
    // verify ring (ring_len > 0): committed-token count per (slot, layer), the
    // ring commit's per-slot group counters (0 between calls) and the token records,
    // ring_stride floats per (slot, layer): k^ [L][h_k][d], v [L][h_v][d],
    // a [L][h_v], b [L][h_v]
    int32_t* ring_cnt;
    int32_t* ring_arr;
    float* ring;
    int64_t ring_stride;
    int32_t ring_len;
    int32_t n_slots, n_layers, h_k, h_v, d, conv_k, c_conv;
    float q_scale, eps;
};

}  // namespace gdn

// Host-side pool object (opaque to callers).
struct gdn_pool {
    gdn_pool_desc desc;
    gdn::PoolView view;
    size_t state_bytes, aux_bytes, window_bytes;
    int io_size;
};

namespace gdn {

// Kernel launchers (defined next to their kernels).  All return hipError_t
// from the launch; arguments were validated by the caller.
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream);
hipError_t launch_slot_reset(const gdn_pool* pool, int32_t n, const int32_t* slot_ids,
                             hipStream_t stream);
hipError_t launch_slot_copy(const gdn_pool* pool, int32_t n, const int32_t* src_ids,
                            const int32_t* dst_ids, hipStream_t stream);
// More than 64 KiB of dynamic LDS has to be enabled per kernel (gfx950 has
// 160 KiB per CU).  Done once per kernel and device: `done` holds one bit per
// device id below 64 (set with release order once the attribute is in
// place; devices from 64 on set it on every call), so concurrent first calls
// from several host threads at worst set the same attribute twice.
template <typename KFn>
hipError_t allow_dynamic_lds(KFn* kernel, size_t bytes, std::atomic<uint64_t>* done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done->load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess && bit) done->fetch_or(bit, std::memory_order_release);
    return e;
}

// Compute units of the current device (queried once per device; 0 if the
// query fails).
inline int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Prefill checkpoints: after every `every_chunks` chunks of sequence j,
// checkpoint m goes to slot slots[off[j] + m] (if m < off[j+1] - off[j]).
struct Ckpt {
    int every_chunks;      // 0: none
    const int32_t* off;    // [n_seq+1]
    const int32_t* slots;  // [off[n_seq]]
};
hipError_t launch_decode_verify(const gdn_pool* pool, int32_t layer, int32_t n,
                                const int32_t* slot_ids, int32_t n_tok, const void* q,
                                const void* k, const void* v, const float* a, const float* b,
                                const float* conv_w, const int32_t* accept_len, void* out,
                                hipStream_t stream);
// Low-batch decode with the rows of each head split over workgroups:
// the split factor for n entries (1 = use the one-workgroup kernel).
int decode_rows_split(const gdn_pool* pool, int32_t n);
// Decode (n_tok = 1, no accept_len) and verify with one value head per
// workgroup (d_k 64 or 128): batches above the row split.
bool decode_heads_ok(const gdn_pool* pool);
hipError_t launch_decode_heads(const gdn_pool* pool, int32_t layer, int32_t n,
                               const int32_t* slot_ids, int32_t n_tok, const void* q,
                               const void* k, const void* v, const float* a, const float* b,
                               const float* conv_w, const int32_t* accept_len, void* out,
                               hipStream_t stream);
hipError_t launch_decode_rows(const gdn_pool* pool, int nrb, int32_t layer, int32_t n,
                              const int32_t* slot_ids, const void* q, const void* k, const void* v,
                              const float* a, const float* b, const float* conv_w, void* out,
                              hipStream_t stream);
// Verify ring (pools with ring_len > 0).
constexpr int kMaxRingSolve = 32;   // ring_len + n_tok
enum class RingOp { kVerify, kCommit, kFlush };
hipError_t launch_ring(const gdn_pool* pool, RingOp op, int32_t layer, int32_t n,
                       const int32_t* slot_ids, int32_t n_tok, const void* q, const void* k,
                       const void* v, const float* a, const float* b, const float* conv_w,
                       const int32_t* accept_len, void* out, hipStream_t stream);
// Input projection y = x W^T with the q | k | v | a | b epilogue.
size_t in_proj_workspace_bytes(const gdn_pool* pool, int64_t n_tok, int32_t hidden);
hipError_t launch_in_proj(const gdn_pool* pool, int64_t n_tok, int32_t hidden, const void* x,
                          const void* w, void* q, void* k, void* v, float* a, float* b,
                          void* workspace, hipStream_t stream);
size_t prefill_workspace_bytes(const gdn_pool* pool, int32_t n_seq, int64_t total_tokens,
                               int32_t chunk);
// The static prefill scratch (kStaticScratchBytes on every device): its
// address on the current device, resolved on the first call there.
constexpr size_t kStaticScratchBytes = GDN_STATIC_SCRATCH_BYTES;
hipError_t prefill_static_scratch(void** ptr);
hipError_t launch_prefill(const gdn_pool* pool, int32_t layer, int32_t n_seq,
                          const int32_t* cu_seqlens, const int32_t* slot_ids,
                          int64_t total_tokens, int32_t chunk, const void* q, const void* k,
                          const void* v, const float* a, const float* b, const float* conv_w,
                          void* out, void* workspace, Ckpt ck, hipStream_t stream);

}  // namespace gdn
