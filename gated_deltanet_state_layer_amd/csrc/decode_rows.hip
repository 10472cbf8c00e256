// Low-batch decode: the rows of each value head split over NRB workgroups.
//
// With few entries the one-workgroup-per-(entry, q/k group) decode runs on
// only n * h_k CUs and is bound by one workgroup's latency (the pages put
// batch-1 GDN decode at about 2 % of HBM: "Plan (research-based):
// Qwen3.6-35B-A3B -- parity fix + path to >150 tok/s", section "Honest
// caveat on speed").  Here workgroup (entry, group, rb) owns
// rows [rb*D/NRB, (rb+1)*D/NRB) of the group's G value-head tiles and the v
// conv channels of those rows, so NRB times more CUs stream the state.  The
// arithmetic per row is that of the one-workgroup kernel (same row split over
// D/8 lanes, same DPP sums and operation order), so outputs and states are
// bitwise equal to it.
//
// Every workgroup of a group needs the group's q^ and k^, so each recomputes
// the q/k conv from the old window.  The q/k window may only roll after all
// of them have read it: each workgroup increments a per-(slot, layer, group)
// counter after its reads, and the one that brings it to NRB rolls the q/k
// window and clears the counter.  Nothing waits on another workgroup.
#include "gdn_common.h"

namespace gdn {
namespace {

constexpr int kRowThreads = 256;   // threads per value head
constexpr int kRowHeads = 2;       // value heads per workgroup (G <= 2)
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kStatePolicy = 2;    // non-temporal: each state row is read and written once

typedef float f32x4 __attribute__((ext_vector_type(4)));

// KC > 0: conv taps fixed at compile time (must equal conv_k); 0: runtime.
template <int D, typename T, int NRB, int KC>
__global__ __launch_bounds__(kRowThreads * kRowHeads) void decode_rows_kernel(
    PoolView P, int layer, const int32_t* __restrict__ slot_ids, const T* __restrict__ q,
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ a,
    const float* __restrict__ b, const float* __restrict__ conv_w, T* __restrict__ out) {
    constexpr int RB = D / NRB;              // rows per head in this workgroup
    constexpr int LPR = D / 8;               // lanes per row
    constexpr int RPP = kRowThreads / LPR;   // rows per pass
    constexpr int NP = (RB + RPP - 1) / RPP;
    extern __shared__ float smem[];
    __shared__ int s_last;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int g = blockIdx.x / NRB, rb = blockIdx.x % NRB;
    const int i = blockIdx.y;
    const int slot = slot_ids[i];
    if (slot < 0) return;   // padding entry
    if (slot >= P.n_slots) {
        if (tid == 0 && rb == 0) atomicOr(P.err, kErrSlotRange);
        return;
    }
    const int G = P.h_v / P.h_k;   // <= kRowHeads (launcher)
    const int K = KC > 0 ? KC : P.conv_k, C = P.c_conv;
    constexpr int KM = KC > 0 ? KC : kMaxConvK;   // compile-time tap bound
    const int nch = 2 * D + G * RB;   // q, k, then the v channels of this block's rows
    // Wave-uniform (kRowThreads is a multiple of 64); said so to the compiler,
    // so the row descriptors live in scalar registers.
    const int sub = __builtin_amdgcn_readfirstlane(tid / kRowThreads), ht = tid % kRowThreads;
    const int lr = ht % LPR, lrow0 = ht / LPR;
    const int c0 = 4 * lr, c1 = D / 2 + 4 * lr;
    const int voff = (lrow0 * D + c0) * (int)sizeof(float);
    constexpr int kSeg1 = D / 2 * (int)sizeof(float);
    constexpr int kPass = RPP * D * (int)sizeof(float);
    const int hv = g * G + sub;
    // This block's rows of value head hv; rows past RB read as zero through
    // the descriptor's range and are never stored.
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        P.state + (((int64_t)slot * P.n_layers + layer) * P.h_v + hv) * (int64_t)D * D +
            (int64_t)rb * RB * D,
        0, RB * D * (int)sizeof(float), kRsrcWord3);
    // LDS: line [K-1][nch] rolled window rows (for the q/k roll), act [nch],
    //      nrm [3], obuf [G][RB] outputs.
    float* line = smem;
    float* act = line + (KM - 1) * nch;
    float* nrm = act + nch;
    float* obuf = nrm + 4;

    // ---- front end: conv + SiLU of q, k and this block's v channels (one
    // channel per thread).  The channel's window rows, token value and
    // weights are all requested before the state rows, so the conv waits for
    // its own loads only.
    T* win = reinterpret_cast<T*>(P.window) + ((int64_t)slot * P.n_layers + layer) * (int64_t)(K - 1) * C;
    const int c = tid;
    const bool has_c = c < nch;
    int gc = 0;
    float xl[KM], wl[KM];
    if (has_c) {
        const T* src;
        if (c < D) {
            gc = g * D + c;
            src = q + ((int64_t)i * P.h_k + g) * D + c;
        } else if (c < 2 * D) {
            gc = P.h_k * D + g * D + (c - D);
            src = k + ((int64_t)i * P.h_k + g) * D + (c - D);
        } else {
            const int hl = (c - 2 * D) / RB, rr = (c - 2 * D) % RB;
            gc = 2 * P.h_k * D + (g * G + hl) * D + rb * RB + rr;
            src = v + ((int64_t)i * P.h_v + g * G + hl) * D + rb * RB + rr;
        }
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            if (j < K - 1) xl[j] = Io<T>::load(win, (int64_t)j * C + gc);
            else if (j == K - 1) xl[j] = Io<T>::load(src, 0);
            else xl[j] = 0.f;
            wl[j] = j < K ? conv_w[(int64_t)gc * K + j] : 0.f;
        }
    }
    float s[NP][8];
    if (sub < G) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const f32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, p * kPass, kStatePolicy);
            const f32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + kSeg1, p * kPass, kStatePolicy);
            s[p][0] = x0.x; s[p][1] = x0.y; s[p][2] = x0.z; s[p][3] = x0.w;
            s[p][4] = x1.x; s[p][5] = x1.y; s[p][6] = x1.z; s[p][7] = x1.w;
        }
    }

    if (has_c) {
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < KM; ++j) z = fmaf(wl[j], xl[j], z);
        act[c] = silu(z);
#pragma unroll
        for (int j = 1; j < KM; ++j) line[(j - 1) * nch + c] = xl[j];   // the rolled window rows
        if (c >= 2 * D)   // this block alone owns these v channels: roll now
#pragma unroll
            for (int r = 0; r < KM - 1; ++r)
                if (r < K - 1) Io<T>::store(win, (int64_t)r * C + gc, xl[r + 1]);
    }
    __syncthreads();
    // Every q/k window read of this workgroup has returned its value (in
    // LDS), so no later store can affect it: count the workgroup now.  The
    // result is only needed at the end, where the last of the NRB workgroups
    // rolls the q/k window (its stores are issued after it saw every other
    // workgroup's increment, hence after all of their reads).
    int32_t* ctr = P.ctr + ((int64_t)slot * P.n_layers + layer) * P.h_k + g;
    int arrived = 0;
    if (tid == 0) arrived = atomicAdd(ctr, 1);
    // ---- q/k normalisation factors and k.q (wave 0).
    if (tid < 64) {
        float sq = 0.f, sk = 0.f, sqk = 0.f;
        for (int c = tid; c < D; c += 64) {
            const float xq = act[c], xk = act[D + c];
            sq = fmaf(xq, xq, sq);
            sk = fmaf(xk, xk, sk);
            sqk = fmaf(xq, xk, sqk);
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        sqk = wave_sum(sqk);
        if (tid == 0) {
            const float rq = P.q_scale / sqrtf(sq + P.eps);
            const float rk = 1.0f / sqrtf(sk + P.eps);
            nrm[0] = rq;
            nrm[1] = rk;
            nrm[2] = sqk * rq * rk;
        }
    }
    __syncthreads();

    // ---- this block's rows of the G value heads (one head per 256 threads).
    if (sub < G) {
        const float rq = nrm[0], rk = nrm[1], kq = nrm[2];
        float kc[8], qc[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qc[e] = act[c0 + e] * rq;
            qc[4 + e] = act[c1 + e] * rq;
            kc[e] = act[D + c0 + e] * rk;
            kc[4 + e] = act[D + c1 + e] * rk;
        }
        const float at = a[(int64_t)i * P.h_v + hv];
        const float bt = b[(int64_t)i * P.h_v + hv];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float u = 0.f, pq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u = fmaf(s[p][e], kc[e], u);
                pq = fmaf(s[p][e], qc[e], pq);
            }
            u = group_sum<LPR>(u);
            pq = group_sum<LPR>(pq);
            const int lrow = lrow0 + p * RPP;
            const float vi = lrow < RB ? act[2 * D + sub * RB + lrow] : 0.f;
            const float delta = bt * (vi - at * u);
#pragma unroll
            for (int e = 0; e < 8; ++e) s[p][e] = fmaf(at, s[p][e], delta * kc[e]);
            if (lr == 0 && lrow < RB) obuf[sub * RB + lrow] = fmaf(at, pq, delta * kq);
            if (lrow < RB) {
                __builtin_amdgcn_raw_buffer_store_b128(f32x4{s[p][0], s[p][1], s[p][2], s[p][3]}, rs,
                                                       voff, p * kPass, kStatePolicy);
                __builtin_amdgcn_raw_buffer_store_b128(f32x4{s[p][4], s[p][5], s[p][6], s[p][7]}, rs,
                                                       voff + kSeg1, p * kPass, kStatePolicy);
            }
        }
    }
    if (tid == 0) s_last = arrived == NRB - 1;
    __syncthreads();
    if (s_last) {   // the last workgroup of the group rolls the q/k window
        for (int e = tid; e < (K - 1) * 2 * D; e += nthr) {
            const int r = e / (2 * D), c = e % (2 * D);
            const int gc = c < D ? g * D + c : P.h_k * D + g * D + (c - D);
            Io<T>::store(win, (int64_t)r * C + gc, line[r * nch + c]);
        }
        if (tid == 0) atomicExch(ctr, 0);
    }
    // ---- outputs: RB contiguous values per head, 16-byte vectors.
    constexpr int VN = 16 / sizeof(T);
    static_assert(RB % VN == 0, "row block must fill whole 16-byte vectors");
    for (int e = tid; e < G * RB / VN; e += nthr) {
        const int hl = e / (RB / VN), j = (e % (RB / VN)) * VN;
        const float* src = obuf + hl * RB + j;
        T* dst = out + ((int64_t)i * P.h_v + g * G + hl) * D + rb * RB + j;
        if constexpr (sizeof(T) == 2) {
            uint4 u;
            u.x = f32_to_bf16(src[0]) | ((uint32_t)f32_to_bf16(src[1]) << 16);
            u.y = f32_to_bf16(src[2]) | ((uint32_t)f32_to_bf16(src[3]) << 16);
            u.z = f32_to_bf16(src[4]) | ((uint32_t)f32_to_bf16(src[5]) << 16);
            u.w = f32_to_bf16(src[6]) | ((uint32_t)f32_to_bf16(src[7]) << 16);
            *reinterpret_cast<uint4*>(dst) = u;
        } else {
            *reinterpret_cast<float4*>(dst) = make_float4(src[0], src[1], src[2], src[3]);
        }
    }
}

template <int D, typename T, int NRB, int KC>
hipError_t launch_rows_k(const gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                         const void* q, const void* k, const void* v, const float* a,
                         const float* b, const float* conv_w, void* out, hipStream_t stream) {
    const PoolView& P = pool->view;
    const int G = P.h_v / P.h_k;
    constexpr int RB = D / NRB;
    constexpr int KM = KC > 0 ? KC : kMaxConvK;
    const int nch = 2 * D + G * RB;   // <= 2D + 2 * D/2 = 3D <= 384 channels
    const size_t lds = ((size_t)(KM - 1) * nch + nch + 4 + G * RB) * sizeof(float);
    // 512 threads whatever G is: one conv channel per thread (2D + G*D/NRB of
    // them), 256 threads per value head for the rows.
    hipLaunchKernelGGL((decode_rows_kernel<D, T, NRB, KC>), dim3(P.h_k * NRB, n),
                       dim3(kRowThreads * kRowHeads), lds, stream, P, layer, slot_ids,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                       a, b, conv_w, static_cast<T*>(out));
    return hipGetLastError();
}

template <int D, typename T, int NRB>
hipError_t launch_rows(const gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                       const void* q, const void* k, const void* v, const float* a, const float* b,
                       const float* conv_w, void* out, hipStream_t stream) {
    if (pool->view.conv_k == 4)
        return launch_rows_k<D, T, NRB, 4>(pool, layer, n, slot_ids, q, k, v, a, b, conv_w, out, stream);
    return launch_rows_k<D, T, NRB, 0>(pool, layer, n, slot_ids, q, k, v, a, b, conv_w, out, stream);
}

template <typename T>
hipError_t launch_rows_t(const gdn_pool* pool, int nrb, int32_t layer, int32_t n,
                         const int32_t* slot_ids, const void* q, const void* k, const void* v,
                         const float* a, const float* b, const float* conv_w, void* out,
                         hipStream_t stream) {
    if (pool->view.d == 128) {
        if (nrb == 8) return launch_rows<128, T, 8>(pool, layer, n, slot_ids, q, k, v, a, b, conv_w, out, stream);
        if (nrb == 4) return launch_rows<128, T, 4>(pool, layer, n, slot_ids, q, k, v, a, b, conv_w, out, stream);
        return launch_rows<128, T, 2>(pool, layer, n, slot_ids, q, k, v, a, b, conv_w, out, stream);
    }
    if (nrb == 4) return launch_rows<64, T, 4>(pool, layer, n, slot_ids, q, k, v, a, b, conv_w, out, stream);
    return launch_rows<64, T, 2>(pool, layer, n, slot_ids, q, k, v, a, b, conv_w, out, stream);
}

}  // namespace

int decode_rows_split(const gdn_pool* pool, int32_t n) {
    const PoolView& P = pool->view;
    if (P.h_v / P.h_k > kRowHeads || (P.d != 128 && P.d != 64)) return 1;
    // Split only while the one-workgroup kernel would leave most CUs idle
    // (measured: at 256 workgroups the split is no longer faster), into up to
    // 512 workgroups.
    const int64_t wgs = (int64_t)n * P.h_k;   // workgroups of the one-workgroup kernel
    if (wgs > 128) return 1;
    const int max_nrb = P.d == 128 ? 8 : 4;
    int nrb = 1;
    while (nrb < max_nrb && wgs * nrb * 2 <= 512) nrb *= 2;
    return nrb;
}

hipError_t launch_decode_rows(const gdn_pool* pool, int nrb, int32_t layer, int32_t n,
                              const int32_t* slot_ids, const void* q, const void* k, const void* v,
                              const float* a, const float* b, const float* conv_w, void* out,
                              hipStream_t stream) {
    if (pool->desc.io_dtype == GDN_BF16)
        return launch_rows_t<uint16_t>(pool, nrb, layer, n, slot_ids, q, k, v, a, b, conv_w, out, stream);
    return launch_rows_t<float>(pool, nrb, layer, n, slot_ids, q, k, v, a, b, conv_w, out, stream);
}

}  // namespace gdn
