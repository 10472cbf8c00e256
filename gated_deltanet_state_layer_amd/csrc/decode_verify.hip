// Multi-slot decode and speculative verify for the gated delta rule.
//
// One workgroup owns one (entry, q/k head group): the conv channels of that
// group (its q head, its k head and the G = h_v/h_k value heads that share
// them) and the G fp32 [d_v][d_k] state tiles of those value heads in the
// entry's slot.  No other workgroup touches these channels or tiles, so the
// in-place conv-window roll and the state write-back need no cross-workgroup
// ordering (baseRT issue #31, "Why this looks tractable": a slot index in the
// recurrence and conv kernels).
//
// The state update is bound by HBM: each tile is read once and written once
// (bytes per slot: 2 * h_v * d_v * d_k * 4).  Each row of a tile is split over
// D/8 lanes holding 8 fp32 columns (two 16-byte loads), so a wave instruction
// moves contiguous 256/128/64-byte row segments.  A row's two dot products
// (S.k and S.q) are summed across its lanes with DPP, then
//     delta = b (v - a S.k),  S <- a S + delta k^T,  o = a S.q + delta k.q
// which is S <- a S (I - b k k^T) + b v k^T and o = S_new q written as one
// pass over the row ("Plan (research-based): Qwen3.6-35B-A3B", "What the
// research found": delta rule over a [V,K] state).
//
// Verify keeps each thread's rows in registers across the n_tok tokens, writes
// every position's output and stores the rows once, after accept_len tokens
// ("Plan (research-based)", "What the research found" and "Why >150 is still
// reachable": no per-position state snapshots).  Decode is the same kernel
// with one token, so verify positions are bitwise equal to decode steps.
// With d_k = 64 or 128 the library runs the head-split kernels of
// decode_rows.hip instead (same arithmetic, bitwise equal); this kernel
// serves the other head sizes.
#include "gdn_common.h"

namespace gdn {
namespace {

constexpr int kHeadThreads = 256;       // threads per value-head tile
constexpr int kMaxHeadsPerBlock = 2;    // value heads streamed concurrently per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The state tiles are streamed with buffer instructions: one descriptor per
// tile (base in scalar registers), one 32-bit lane offset, and the per-pass
// row offset in a scalar register, so a lane needs no per-row addresses.
// Cache policy: loads default, stores non-temporal (each tile is read once
// and written once).  Measured at 64 slots: non-temporal loads and stores
// 54.3 us, default loads 53.7 us, default stores 60.7 us, both default
// 68.5 us; verify 110.8 -> 108.2 us with default loads.
constexpr int kStateLoadPolicy = 0;
constexpr int kStateStorePolicy = 2;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(float* tile, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(tile, 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ f32x4 ld_state(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStateLoadPolicy);
}
__device__ __forceinline__ void st_state(__amdgpu_buffer_rsrc_t r, int voff, int soff, f32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(x, r, voff, soff, kStateStorePolicy);
}

// NTOK > 0: token count fixed at compile time (decode: 1); 0: runtime (verify).
template <int D, typename T, int NTOK>
__global__ __launch_bounds__(kHeadThreads * kMaxHeadsPerBlock) void decode_verify_kernel(
    PoolView P, int layer, const int32_t* __restrict__ slot_ids, int n_tok_rt,
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, const float* __restrict__ conv_w,
    const int32_t* __restrict__ accept_len, T* __restrict__ out) {
    extern __shared__ float smem[];
    const int n_tok = NTOK > 0 ? NTOK : n_tok_rt;
    const int nthr = blockDim.x;
    const int tid = threadIdx.x;
    const int g = blockIdx.x;   // q/k head group
    const int i = blockIdx.y;   // entry
    const int slot = slot_ids[i];
    if (slot < 0) return;  // padding entry
    if (slot >= P.n_slots) {
        if (tid == 0) atomicOr(P.err, kErrSlotRange);
        return;
    }
    const int G = P.h_v / P.h_k;
    const int HB = nthr / kHeadThreads;   // heads per round
    const int K = P.conv_k;
    const int C = P.c_conv;
    const int nch = (2 + G) * D;  // channels owned by this group
    int commit = n_tok;
    if (accept_len) commit = min(max(accept_len[i], 0), n_tok);
    // Without outputs (commit only) the tokens after accept_len are not run.
    const int t_end = NTOK > 0 ? NTOK : (out ? n_tok : commit);

    // ---- state tile mapping: each row split over LPR lanes, 8 columns per
    // lane (two 16-byte segments, D/2 apart); RPP rows per pass.
    constexpr int LPR = D / 8;
    constexpr int RPP = kHeadThreads / LPR;
    constexpr int NP = (D + RPP - 1) / RPP;
    // Wave-uniform (a tile is a whole number of waves); said so to the
    // compiler, so the tile descriptors live in scalar registers.
    const int sub = __builtin_amdgcn_readfirstlane(tid / kHeadThreads);
    const int ht = tid % kHeadThreads;
    const int lr = ht % LPR;
    const int row0 = ht / LPR;
    const int c0 = 4 * lr, c1 = D / 2 + 4 * lr;
    const int voff = (row0 * D + c0) * (int)sizeof(float);   // byte offset of pass 0, segment 0
    constexpr int kSeg1 = D / 2 * (int)sizeof(float);         // segment 1, immediate offset
    constexpr int kPass = RPP * D * (int)sizeof(float);       // bytes between passes
    constexpr int kTileBytes = D * D * (int)sizeof(float);
    float* slot_state = P.state + ((int64_t)slot * P.n_layers + layer) * (int64_t)P.h_v * D * D;

    float s[NP][8];
    // Rows past D (only when D < RPP) read as zero through the descriptor's
    // range check and are never stored.
    auto load_tile = [&](__amdgpu_buffer_rsrc_t rs) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const f32x4 x0 = ld_state(rs, voff, p * kPass);
            const f32x4 x1 = ld_state(rs, voff + kSeg1, p * kPass);
            s[p][0] = x0.x; s[p][1] = x0.y; s[p][2] = x0.z; s[p][3] = x0.w;
            s[p][4] = x1.x; s[p][5] = x1.y; s[p][6] = x1.z; s[p][7] = x1.w;
        }
    };
    // LDS: line [K-1+n_tok][nch] raw inputs (window rows, then tokens),
    //      act  [n_tok][nch]     conv+SiLU outputs,
    //      nrm  [n_tok][3]       q scale, k scale, k.q
    //      gate [2][n_tok][G]    a, then b, of the group's value heads
    //      obuf [n_tok][G][D]    outputs, over `line` once the front end is done
    const int L = K - 1 + n_tok;
    float* line = smem;
    float* act = line + L * nch;
    float* nrm = act + n_tok * nch;
    float* gate = nrm + n_tok * 3;
    const int ngate = 2 * n_tok * G;
    // Gate e of the staged set: a (e < n_tok*G) or b, token t, group head hl.
    const auto gate_src = [&](int e) {
        const int which = e >= n_tok * G, rem = which ? e - n_tok * G : e;
        return (which ? b : a) + ((int64_t)i * n_tok + rem / G) * P.h_v + g * G + rem % G;
    };
    float* obuf = line;   // [n_tok][G][D] outputs; reuses `line` after the front end
    T* win = reinterpret_cast<T*>(P.window) +
             ((int64_t)slot * P.n_layers + layer) * (int64_t)(K - 1) * C;
    const auto first_tiles = [&]() {
        if (sub < G) load_tile(tile_rsrc(slot_state + (int64_t)(g * G + sub) * D * D, kTileBytes));
    };

    // ---- front end: depthwise causal conv + SiLU over the group's channels.
    // Verify in the common shape (conv_k = 4, one channel per thread, at most
    // kFastTok tokens): the raw inputs are loaded into registers first and the
    // state tiles after them, so the conv waits only for its own data while
    // the state streams in (loads complete in order).  Otherwise, and for
    // decode (measured slightly faster that way), the state loads go first
    // and the conv follows from LDS.
    constexpr int kFastTok = 4;
    const float graw = *gate_src(min(tid, ngate - 1));   // issued ahead of the state
    const bool fast = NTOK == 0 && K == 4 && nch <= nthr && n_tok <= kFastTok;   // uniform
    if (fast) {
        const int c = min(tid, nch - 1);
        int gc;
        const T* src;
        int64_t tstride;
        if (c < D) {
            gc = g * D + c;
            src = q + ((int64_t)i * n_tok * P.h_k + g) * D + c;
            tstride = (int64_t)P.h_k * D;
        } else if (c < 2 * D) {
            gc = P.h_k * D + g * D + (c - D);
            src = k + ((int64_t)i * n_tok * P.h_k + g) * D + (c - D);
            tstride = (int64_t)P.h_k * D;
        } else {
            gc = 2 * P.h_k * D + g * G * D + (c - 2 * D);
            src = v + ((int64_t)i * n_tok * P.h_v + g * G) * D + (c - 2 * D);
            tstride = (int64_t)P.h_v * D;
        }
        constexpr int NX = 3 + kFastTok;
        T rx[NX];
        float wc[4];
#pragma unroll
        for (int r = 0; r < 3; ++r) rx[r] = win[(int64_t)r * C + gc];
#pragma unroll
        for (int t = 0; t < kFastTok; ++t) rx[3 + t] = src[(t < n_tok ? t : 0) * tstride];
#pragma unroll
        for (int j = 0; j < 4; ++j) wc[j] = conv_w[(int64_t)gc * 4 + j];
        first_tiles();
        asm volatile("" ::: "memory");   // keep the state loads after the conv inputs
        if (tid < nch) {
            // Same accumulation order as the general loop below, so decode
            // and verify positions stay bitwise equal.
#pragma unroll
            for (int t = 0; t < kFastTok; ++t) {
                if (t < n_tok) {
                    float z = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) z = fmaf(wc[j], Io<T>::load(rx, t + j), z);
                    act[t * nch + c] = silu(z);
                }
            }
            // Roll the window by `commit` tokens: row r takes input commit + r.
            if (commit > 0) {
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    T x = rx[r + 1];
#pragma unroll
                    for (int m = 2; m <= kFastTok; ++m)
                        if (commit == m) x = rx[r + m];
                    win[(int64_t)r * C + gc] = x;
                }
            }
        }
    } else {
        // Issue the first round's state loads before the conv front end so the
        // HBM stream overlaps it.
        first_tiles();
    }
    for (int c = fast ? nch : tid; c < nch; c += nthr) {
        int gc;             // global channel
        const T* src;       // token 0 of this channel
        int64_t tstride;    // element stride between tokens
        if (c < D) {
            gc = g * D + c;
            src = q + ((int64_t)i * n_tok * P.h_k + g) * D + c;
            tstride = (int64_t)P.h_k * D;
        } else if (c < 2 * D) {
            gc = P.h_k * D + g * D + (c - D);
            src = k + ((int64_t)i * n_tok * P.h_k + g) * D + (c - D);
            tstride = (int64_t)P.h_k * D;
        } else {
            gc = 2 * P.h_k * D + g * G * D + (c - 2 * D);
            src = v + ((int64_t)i * n_tok * P.h_v + g * G) * D + (c - 2 * D);
            tstride = (int64_t)P.h_v * D;
        }
        for (int r = 0; r < K - 1; ++r) line[r * nch + c] = Io<T>::load(win, (int64_t)r * C + gc);
        for (int t = 0; t < n_tok; ++t) line[(K - 1 + t) * nch + c] = Io<T>::load(src, t * tstride);
        const float* wc = conv_w + (int64_t)gc * K;
        for (int t = 0; t < n_tok; ++t) {
            float z = 0.f;
            for (int j = 0; j < K; ++j) z = fmaf(wc[j], line[(t + j) * nch + c], z);
            act[t * nch + c] = silu(z);
        }
        // Roll the window by `commit` tokens (same thread, after all reads).
        if (commit > 0)
            for (int r = 0; r < K - 1; ++r)
                Io<T>::store(win, (int64_t)r * C + gc, line[(commit + r) * nch + c]);
    }
    if (tid < ngate) gate[tid] = graw;
    for (int e = tid + nthr; e < ngate; e += nthr) gate[e] = *gate_src(e);
    __syncthreads();

    // ---- q/k normalisation factors and k.q per token (one wave per token).
    {
        const int wave = tid >> 6, lane = tid & 63;
        for (int t = wave; t < n_tok; t += nthr / 64) {
            float sq = 0.f, sk = 0.f, sqk = 0.f;
            for (int c = lane; c < D; c += 64) {
                const float xq = act[t * nch + c], xk = act[t * nch + D + c];
                sq = fmaf(xq, xq, sq);
                sk = fmaf(xk, xk, sk);
                sqk = fmaf(xq, xk, sqk);
            }
            sq = wave_sum(sq);
            sk = wave_sum(sk);
            sqk = wave_sum(sqk);
            if (lane == 0) {
                const float rq = P.q_scale / sqrtf(sq + P.eps);
                const float rk = 1.0f / sqrtf(sk + P.eps);
                nrm[t * 3 + 0] = rq;
                nrm[t * 3 + 1] = rk;
                nrm[t * 3 + 2] = sqk * rq * rk;
            }
        }
    }
    __syncthreads();

    // ---- state tiles, HB value heads at a time.
    for (int r = 0;; ++r) {
        const int hl = r * HB + sub;
        if (hl >= G) break;
        const int hv = g * G + hl;
        const __amdgpu_buffer_rsrc_t rs = tile_rsrc(slot_state + (int64_t)hv * D * D, kTileBytes);
        if (r > 0) load_tile(rs);
        for (int t = 0; t < t_end; ++t) {
            const float* y = act + t * nch;
            const float rq = nrm[t * 3 + 0], rk = nrm[t * 3 + 1], kq = nrm[t * 3 + 2];
            float kc[8], qc[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qc[e] = y[c0 + e] * rq;
                qc[4 + e] = y[c1 + e] * rq;
                kc[e] = y[D + c0 + e] * rk;
                kc[4 + e] = y[D + c1 + e] * rk;
            }
            const float at = gate[t * G + hl];
            const float bt = gate[(n_tok + t) * G + hl];
            float* o_row = obuf + (t * G + hl) * D;
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
                const int row = row0 + p * RPP;
                const float vi = (row < D) ? y[2 * D + hl * D + row] : 0.f;
                const float delta = bt * (vi - at * u);
#pragma unroll
                for (int e = 0; e < 8; ++e) s[p][e] = fmaf(at, s[p][e], delta * kc[e]);
                if (lr == 0 && row < D) o_row[row] = fmaf(at, pq, delta * kq);
                if (t + 1 == commit && row < D) {
                    st_state(rs, voff, p * kPass, f32x4{s[p][0], s[p][1], s[p][2], s[p][3]});
                    st_state(rs, voff + kSeg1, p * kPass, f32x4{s[p][4], s[p][5], s[p][6], s[p][7]});
                }
            }
        }
    }

    // ---- outputs: staged in LDS, written as 16-byte vectors (for each token
    // the group's G value heads are contiguous in `out`).
    __syncthreads();
    if (out) {
        constexpr int VN = 16 / sizeof(T);
        const int nvec = n_tok * G * D / VN;
        for (int e = tid; e < nvec; e += nthr) {
            const int t = e / (G * D / VN), c = (e % (G * D / VN)) * VN;
            const float* src = obuf + t * G * D + c;
            T* dst = out + (((int64_t)i * n_tok + t) * P.h_v + g * G) * D + c;
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
}

size_t lds_bytes(const PoolView& P, int n_tok) {
    const int G = P.h_v / P.h_k;
    return (size_t)(P.conv_k - 1 + 2 * n_tok) * (2 + G) * P.d * sizeof(float) +
           (size_t)n_tok * (3 + 2 * G) * sizeof(float);
}

template <int D, typename T>
hipError_t launch_dv(const gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                     int32_t n_tok, const void* q, const void* k, const void* v, const float* a,
                     const float* b, const float* conv_w, const int32_t* accept_len, void* out,
                     hipStream_t stream) {
    const PoolView& P = pool->view;
    const int G = P.h_v / P.h_k;
    const int threads = kHeadThreads * (G < kMaxHeadsPerBlock ? G : kMaxHeadsPerBlock);
    const size_t lds = lds_bytes(P, n_tok);
    dim3 grid(P.h_k, n);
    const T* qq = static_cast<const T*>(q);
    const T* kk = static_cast<const T*>(k);
    const T* vv = static_cast<const T*>(v);
    T* oo = static_cast<T*>(out);
    if (n_tok == 1)
        hipLaunchKernelGGL((decode_verify_kernel<D, T, 1>), grid, dim3(threads), lds, stream, P,
                           layer, slot_ids, 1, qq, kk, vv, a, b, conv_w, accept_len, oo);
    else
        hipLaunchKernelGGL((decode_verify_kernel<D, T, 0>), grid, dim3(threads), lds, stream, P,
                           layer, slot_ids, n_tok, qq, kk, vv, a, b, conv_w, accept_len, oo);
    return hipGetLastError();
}

}  // namespace

size_t decode_verify_lds_bytes(const gdn_pool* pool, int32_t n_tok) {
    return lds_bytes(pool->view, n_tok);
}

hipError_t launch_decode_verify(const gdn_pool* pool, int32_t layer, int32_t n,
                                const int32_t* slot_ids, int32_t n_tok, const void* q,
                                const void* k, const void* v, const float* a, const float* b,
                                const float* conv_w, const int32_t* accept_len, void* out,
                                hipStream_t stream) {
    const bool bf = pool->desc.io_dtype == GDN_BF16;
    switch (pool->view.d) {
#define GDN_CASE(DD)                                                                             \
    case DD:                                                                                     \
        return bf ? launch_dv<DD, uint16_t>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b,      \
                                            conv_w, accept_len, out, stream)                     \
                  : launch_dv<DD, float>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w, \
                                         accept_len, out, stream);
        GDN_CASE(32)
        GDN_CASE(64)
        GDN_CASE(128)
#undef GDN_CASE
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace gdn
