// Input projection in front of the conv: y = x W^T over the hidden size, for
// a batch of tokens, written straight into the raw q, k, v the other calls
// take and the two gates a = exp(-softplus(y_a)) = 1 / (1 + e^y_a) and
// b = sigmoid(y_b) ("baseRT issue #31", section "Why this looks tractable":
// an input-projection kernel sits beside the conv in the layer's kernels).
// W's rows are the output channels, in the order q heads | k heads | v heads
// | h_v a logits | h_v b logits; x and W are bf16, products are exact in fp32
// and accumulate in fp32 on the bf16 matrix cores.
//
// gemm kernel: grid (N/64, M/64, ksplit), 4 waves; wave w owns 16 output
// channels and the block's 64 tokens (4 MFMA tiles) over its share of the
// hidden dimension.  Both operands come straight from memory into MFMA
// registers: lane (m, q) of an operand reads the 16 bytes of row m at
// k = 8q..8q+7 of the step, so no LDS staging is needed, and buffer
// descriptors return zeros for rows past the ends (ragged token and channel
// counts).  With few tokens the hidden dimension is split over ksplit
// workgroups so that enough weight bytes are in flight; a second kernel adds
// the partial sums.  Otherwise the gemm kernel writes the outputs itself.
#include <algorithm>

#include "gdn_common.h"
#include "mfma_split.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kOffOOB = 0x7fff0000;   // an offset past every descriptor used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ bf16x8 ld_frag(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

struct ProjOut {
    void *q, *k, *v;
    float *a, *b;
    int hkd, hvd, c_conv, h_v, n_out;
};

// Output channel n of token m: a raw q/k/v value or an activated gate.
template <typename T>
__device__ __forceinline__ void put(const ProjOut& o, int64_t m, int n, float y) {
    if (n < o.hkd) Io<T>::store(static_cast<T*>(o.q), m * o.hkd + n, y);
    else if (n < 2 * o.hkd) Io<T>::store(static_cast<T*>(o.k), m * o.hkd + n - o.hkd, y);
    else if (n < o.c_conv) Io<T>::store(static_cast<T*>(o.v), m * o.hvd + n - 2 * o.hkd, y);
    else if (n < o.c_conv + o.h_v) o.a[m * o.h_v + n - o.c_conv] = 1.0f / (1.0f + __expf(y));
    else o.b[m * o.h_v + n - o.c_conv - o.h_v] = 1.0f / (1.0f + __expf(-y));
}

template <typename T>
__global__ __launch_bounds__(kThreads) void in_proj_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int M, int H, ProjOut o,
    float* __restrict__ part, int steps_per_split) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m16 = lane & 15, q4 = lane >> 4;
    const int N = o.n_out;
    const int n0 = (blockIdx.x * 4 + wave) * 16, m0 = blockIdx.y * 64;
    const int nsteps = H / 32;
    const int s_begin = blockIdx.z * steps_per_split;
    const int s_end = min(nsteps, s_begin + steps_per_split);
    const auto x_rs = buf_rsrc(x, M * H * 2), w_rs = buf_rsrc(w, N * H * 2);
    // byte offsets of this lane's 16 bytes at step 0 (rows past the ends read zeros)
    const int w_off = (n0 + m16) * H * 2 + q4 * 16;
    int x_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x_off[i] = (m0 + i * 16 + m16) * H * 2 + q4 * 16;
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // one step ahead: the next step's fragments load while this step multiplies
    auto fetch = [&](int s, bf16x8* xf, bf16x8& wf) {
        const bool ok = s < s_end;
        wf = ld_frag(w_rs, ok ? w_off + s * 64 : kOffOOB);
#pragma unroll
        for (int i = 0; i < 4; ++i) xf[i] = ld_frag(x_rs, ok ? x_off[i] + s * 64 : kOffOOB);
    };
    bf16x8 xa[4], xb[4], wa, wb;
    fetch(s_begin, xa, wa);
    for (int s = s_begin; s < s_end; s += 2) {
        fetch(s + 1, xb, wb);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[i], wa, acc[i], 0, 0, 0);
        fetch(s + 2, xa, wa);
        if (s + 1 < s_end) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[i], wb, acc[i], 0, 0, 0);
        }
    }
    // lane holds y[m0 + 16 i + 4 q + j][n0 + m16]
    const int n = n0 + m16;
    if (n >= N) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + i * 16 + q4 * 4 + j;
            if (m >= M) continue;
            if (part) part[((int64_t)blockIdx.z * M + m) * N + n] = acc[i][j];
            else put<T>(o, m, n, acc[i][j]);
        }
}

// Sum of the ksplit partial products, then the outputs.
template <typename T>
__global__ __launch_bounds__(kThreads) void in_proj_epilogue_kernel(const float* __restrict__ part,
                                                                    int M, int ksplit, ProjOut o) {
    const int64_t total = (int64_t)M * o.n_out;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        float y = 0.f;
        for (int z = 0; z < ksplit; ++z) y += part[z * total + i];
        put<T>(o, i / o.n_out, (int)(i % o.n_out), y);
    }
}

}  // namespace

// Split of the hidden dimension for M tokens: enough workgroups to keep the
// weight stream busy, at least 4 steps of 32 per split.
int in_proj_ksplit(const gdn_pool* pool, int64_t M, int32_t H) {
    const int N = pool->view.c_conv + 2 * pool->view.h_v;
    const int64_t tiles = (int64_t)((N + 63) / 64) * ((M + 63) / 64);
    int ks = (int)std::min<int64_t>(16, std::max<int64_t>(1, 1024 / std::max<int64_t>(tiles, 1)));
    ks = std::min(ks, std::max(1, H / 32 / 4));
    return ks;
}

size_t in_proj_workspace_bytes(const gdn_pool* pool, int64_t M, int32_t H) {
    const int ks = in_proj_ksplit(pool, M, H);
    return ks > 1 ? (size_t)ks * M * (pool->view.c_conv + 2 * pool->view.h_v) * sizeof(float) : 0;
}

hipError_t launch_in_proj(const gdn_pool* pool, int64_t M, int32_t H, const void* x, const void* w,
                          void* q, void* k, void* v, float* a, float* b, void* workspace,
                          hipStream_t stream) {
    const PoolView& P = pool->view;
    ProjOut o{q, k, v, a, b, P.h_k * P.d, P.h_v * P.d, P.c_conv, P.h_v, P.c_conv + 2 * P.h_v};
    const int ks = in_proj_ksplit(pool, M, H);
    const int nsteps = H / 32, per = (nsteps + ks - 1) / ks;
    float* part = ks > 1 ? static_cast<float*>(workspace) : nullptr;
    const dim3 grid((o.n_out + 63) / 64, (unsigned)((M + 63) / 64), ks);
    const auto* xs = static_cast<const uint16_t*>(x);
    const auto* ws = static_cast<const uint16_t*>(w);
    if (pool->desc.io_dtype == GDN_BF16)
        hipLaunchKernelGGL(in_proj_gemm_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, xs, ws,
                           (int)M, H, o, part, per);
    else
        hipLaunchKernelGGL(in_proj_gemm_kernel<float>, grid, dim3(kThreads), 0, stream, xs, ws,
                           (int)M, H, o, part, per);
    if (ks > 1) {
        const int64_t total = M * o.n_out;
        const unsigned blocks = (unsigned)std::min<int64_t>(4096, (total + kThreads - 1) / kThreads);
        if (pool->desc.io_dtype == GDN_BF16)
            hipLaunchKernelGGL(in_proj_epilogue_kernel<uint16_t>, dim3(blocks), dim3(kThreads), 0,
                               stream, part, (int)M, ks, o);
        else
            hipLaunchKernelGGL(in_proj_epilogue_kernel<float>, dim3(blocks), dim3(kThreads), 0,
                               stream, part, (int)M, ks, o);
    }
    return hipGetLastError();
}

}  // namespace gdn
