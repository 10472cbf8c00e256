// Decode and verify split finer than one workgroup per (entry, q/k group):
// the rows of each value head over NRB workgroups for low-batch decode, and
// one workgroup per value head for larger batches and for verify.
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
// The head-split kernel loads its tile with the default policy (stores stay
// non-temporal): 64 of 256 slots took 52.5 us, against 52.95 us with
// non-temporal loads and 54.2 us for the one-workgroup-per-group kernel
// (same-box A/B, two passes).
constexpr int kHeadLoadPolicy = 0;
constexpr int kHeadDecodeOrder = 2;
constexpr int kHeadVerifyOrder = 0;

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

// Decode and verify with one value head per workgroup (batches too large
// for the row split).  Workgroup (head hv, entry i) streams the whole [D][D]
// tile of its head with 256 threads, the tile layout of the one-workgroup
// kernel (a row over D/8 lanes, eight columns each), default-policy loads
// and non-temporal stores.
// It recomputes its group's q^/k^ from the old window (cheap) and owns the v
// channels of its head; the q/k window of the group is rolled by the last of
// its G workgroups to arrive, as in the row split.  DECODE: one token, no
// accept_len; else n_tok <= NB verify tokens (rows kept in registers over the
// tokens, stored once after accept_len of them; every position's output
// written, or none with out = NULL, when the tokens past accept_len are not
// run).  NB, the compile-time token bound, sizes the register arrays.  The
// arithmetic per row, token and channel is that of the one-workgroup kernel,
// so results are bitwise equal to it.
template <int D, typename T, int KC, int NB, bool DECODE>
__global__ __launch_bounds__(kRowThreads) void decode_heads_kernel(
    PoolView P, int layer, const int32_t* __restrict__ slot_ids, int n_tok_rt,
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, const float* __restrict__ conv_w,
    const int32_t* __restrict__ accept_len, T* __restrict__ out) {
    constexpr int LPR = D / 8;               // lanes per row
    constexpr int RPP = kRowThreads / LPR;   // rows per pass
    constexpr int NP = D / RPP;
    constexpr int NCH = 3 * D;               // q, k, then this head's v channels
    constexpr int CPT = (NCH + kRowThreads - 1) / kRowThreads;
    constexpr int KM = KC > 0 ? KC : kMaxConvK;   // compile-time tap bound
    constexpr int NTM = DECODE ? 1 : NB;     // token bound
    constexpr int NX = KM - 1 + NTM;         // raw inputs per channel: window, tokens
    static_assert(CPT * kRowThreads - NCH <= D, "spare threads map onto q channels");
    const auto dup_channel = [](int c) { return c < NCH ? c : c - NCH; };
    extern __shared__ float smem[];
    __shared__ int s_last;
    const int tid = threadIdx.x;
    const int hv = blockIdx.x, i = blockIdx.y;
    const int slot = slot_ids[i];
    if (slot < 0) return;   // padding entry
    if (slot >= P.n_slots) {
        if (tid == 0) atomicOr(P.err, kErrSlotRange);
        return;
    }
    const int n_tok = DECODE ? 1 : n_tok_rt;
    const int commit =
        DECODE ? 1 : (accept_len ? min(max(accept_len[i], 0), n_tok) : n_tok);
    // Without outputs (commit only) the tokens after accept_len are not run.
    const int t_end = DECODE ? 1 : (out ? n_tok : commit);
    const int G = P.h_v / P.h_k, g = hv / G;
    const int K = KC > 0 ? KC : P.conv_k, C = P.c_conv;
    const int lr = tid % LPR, lrow0 = tid / LPR;
    const int c0 = 4 * lr, c1 = D / 2 + 4 * lr;
    const int voff = (lrow0 * D + c0) * (int)sizeof(float);
    constexpr int kSeg1 = D / 2 * (int)sizeof(float);
    constexpr int kPass = RPP * D * (int)sizeof(float);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        P.state + (((int64_t)slot * P.n_layers + layer) * P.h_v + hv) * (int64_t)D * D, 0,
        D * D * (int)sizeof(float), kRsrcWord3);
    // LDS: line [K-1][2D] rolled q/k window rows, act [NTM][3D],
    //      nrm [NTM][8] (q scale, k scale, k.q, a, b), obuf [NTM][D] outputs.
    float* line = smem;
    float* act = line + (KM - 1) * 2 * D;
    float* nrm = act + NTM * NCH;
    float* obuf = nrm + 8 * NTM;

    // ---- front end: conv + SiLU of q, k and this head's v channels, in
    // three groups (front-end loads, state loads, conv) whose order is set
    // below.  The front-end loads are unconditional (token indexes are
    // clamped, and threads past the last channel redo a q channel: its
    // window is written only after every workgroup of the group has read it,
    // while a v channel's window may already be rolled by another wave), so
    // the compiler has no branch to move the conv into.
    T* win = reinterpret_cast<T*>(P.window) + ((int64_t)slot * P.n_layers + layer) * (int64_t)(K - 1) * C;
    T xl[CPT][NX];   // raw index r: window row r (r < K-1), then token r - (K-1)
    float wl[CPT][KM];
    int gcs[CPT];
    float s[NP][8];
    // Verify gates: thread 2t + w < 2 n_tok loads a (w = 0) or b (w = 1) of
    // token t, for LDS.  (Decode reads its two gates as scalars later.)
    const int gt = min(tid >> 1, n_tok - 1), gw = tid & 1;
    float graw = 0.f;
    const auto load_front = [&]() {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c = dup_channel(tid + u * kRowThreads);
            const bool isq = c < D, isk = !isq && c < 2 * D;
            const int cl = c - (isq ? 0 : isk ? D : 2 * D);   // channel within its head
            gcs[u] = isq ? g * D + cl : isk ? P.h_k * D + g * D + cl : 2 * P.h_k * D + hv * D + cl;
            const T* src = isq   ? q + ((int64_t)i * n_tok * P.h_k + g) * D + cl
                           : isk ? k + ((int64_t)i * n_tok * P.h_k + g) * D + cl
                                 : v + ((int64_t)i * n_tok * P.h_v + hv) * D + cl;
            const int64_t tstride = (int64_t)(isq || isk ? P.h_k : P.h_v) * D;
#pragma unroll
            for (int r = 0; r < NX; ++r)
                xl[u][r] = r < K - 1 ? win[(int64_t)r * C + gcs[u]]
                                     : src[min(r - (K - 1), n_tok - 1) * tstride];
#pragma unroll
            for (int j = 0; j < KM; ++j) wl[u][j] = conv_w[(int64_t)gcs[u] * K + min(j, K - 1)];
        }
        if (!DECODE) graw = (gw ? b : a)[((int64_t)i * n_tok + gt) * P.h_v + hv];
    };
    const auto load_state = [&]() {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const f32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, p * kPass, kHeadLoadPolicy);
            const f32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + kSeg1, p * kPass, kHeadLoadPolicy);
            s[p][0] = x0.x; s[p][1] = x0.y; s[p][2] = x0.z; s[p][3] = x0.w;
            s[p][4] = x1.x; s[p][5] = x1.y; s[p][6] = x1.z; s[p][7] = x1.w;
        }
    };
    const auto conv_front = [&]() {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int c = tid + u * kRowThreads;
            // Threads past the last channel compute and store a q channel's
            // value again (the same bits): no branch around the conv.
#pragma unroll
            for (int t = 0; t < NTM; ++t) {
                if (t < n_tok) {
                    float z = 0.f;
#pragma unroll
                    for (int j = 0; j < KM; ++j)
                        if (j < K) z = fmaf(wl[u][j], Io<T>::load(xl[u], t + j), z);
                    act[t * NCH + dup_channel(c)] = silu(z);
                }
            }
            if (c < NCH) {
                // The window advanced by `commit` tokens: row r takes raw input
                // commit + r (selected without a runtime register index).
                T xr[KM - 1];
#pragma unroll
                for (int r = 0; r < KM - 1; ++r) {
                    xr[r] = xl[u][r];
#pragma unroll
                    for (int m = 1; m <= NTM; ++m)
                        if (commit == m) xr[r] = xl[u][r + m];
                }
                if (c < 2 * D) {   // q/k: rolled by the last workgroup of the group
#pragma unroll
                    for (int r = 0; r < KM - 1; ++r)
                        if (r < K - 1) line[r * 2 * D + c] = Io<T>::load(xr, r);
                } else if (commit > 0) {   // v: owned by this workgroup, rolled now
#pragma unroll
                    for (int r = 0; r < KM - 1; ++r)
                        if (r < K - 1) win[(int64_t)r * C + gcs[u]] = xr[r];
                }
            }
        }
    };
    // Order of the three groups, measured on a Qwen3-Next layer: decode of 64
    // of 256 slots is fastest with the state requested first (order 2: 50.6
    // us, against 56.5 us for order 0 and 57.5 us for order 1); verify of 4
    // tokens at 128 slots with the front-end loads first and the conv
    // overlapping the state's arrival (order 0: 101-102.5 us, against
    // 103-105 us for order 1 and 106-108 us for order 2).  The scheduling
    // barriers keep the compiler from moving arithmetic or loads across the
    // groups.
    constexpr int ORDER = DECODE ? kHeadDecodeOrder : kHeadVerifyOrder;
    if constexpr (ORDER == 0) {
        load_front();
        __builtin_amdgcn_sched_barrier(0);
        load_state();
        __builtin_amdgcn_sched_barrier(0);
        conv_front();
    } else if constexpr (ORDER == 1) {
        load_front();
        conv_front();
        __builtin_amdgcn_sched_barrier(0);
        load_state();
    } else {
        load_state();
        __builtin_amdgcn_sched_barrier(0);
        load_front();
        conv_front();
    }
    if (!DECODE && tid < 2 * n_tok) nrm[gt * 8 + 3 + gw] = graw;
    __syncthreads();
    // Every q/k window read of this workgroup has returned (its values are in
    // LDS), so it is counted now; the last of the group's G workgroups rolls
    // the q/k window at the end, after it has seen every other increment.
    int32_t* ctr = P.ctr + ((int64_t)slot * P.n_layers + layer) * P.h_k + g;
    int arrived = 0;
    if (tid == 0) arrived = atomicAdd(ctr, 1);
    // ---- q/k normalisation factors and k.q, one wave per token.
    {
        const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
        for (int t0 = 0; t0 < NTM; t0 += kRowThreads / 64) {
            const int t = t0 + wave;
            if (t >= n_tok) break;
            float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
            for (int c = lane; c < D; c += 64) {
                const float xq = act[t * NCH + c], xk = act[t * NCH + D + c];
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
                nrm[t * 8 + 0] = rq;
                nrm[t * 8 + 1] = rk;
                nrm[t * 8 + 2] = sqk * rq * rk;
            }
        }
    }
    __syncthreads();

    // ---- the head's rows, token by token; stored after `commit` tokens.
    // (A loop the compiler does not unroll: unrolled over the token bound it
    // held more registers.)
#pragma unroll 1
    for (int t = 0; t < t_end; ++t) {
        {
            const float* y = act + t * NCH;
            const float rq = nrm[t * 8 + 0], rk = nrm[t * 8 + 1], kq = nrm[t * 8 + 2];
            float kc[8], qc[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qc[e] = y[c0 + e] * rq;
                qc[4 + e] = y[c1 + e] * rq;
                kc[e] = y[D + c0 + e] * rk;
                kc[4 + e] = y[D + c1 + e] * rk;
            }
            const float at = DECODE ? a[(int64_t)i * P.h_v + hv] : nrm[t * 8 + 3];
            const float bt = DECODE ? b[(int64_t)i * P.h_v + hv] : nrm[t * 8 + 4];
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
                const int row = lrow0 + p * RPP;
                const float vi = y[2 * D + row];
                const float delta = bt * (vi - at * u);
#pragma unroll
                for (int e = 0; e < 8; ++e) s[p][e] = fmaf(at, s[p][e], delta * kc[e]);
                if (lr == 0) obuf[t * D + row] = fmaf(at, pq, delta * kq);
                if (DECODE) {   // each pass stored as soon as it is done
                    __builtin_amdgcn_raw_buffer_store_b128(f32x4{s[p][0], s[p][1], s[p][2], s[p][3]}, rs,
                                                           voff, p * kPass, kStatePolicy);
                    __builtin_amdgcn_raw_buffer_store_b128(f32x4{s[p][4], s[p][5], s[p][6], s[p][7]}, rs,
                                                           voff + kSeg1, p * kPass, kStatePolicy);
                }
            }
            // Verify: one uniform branch after the passes (a branch inside the
            // pass loop would keep the passes from overlapping).
            if (!DECODE && t + 1 == commit) {
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    __builtin_amdgcn_raw_buffer_store_b128(f32x4{s[p][0], s[p][1], s[p][2], s[p][3]}, rs,
                                                           voff, p * kPass, kStatePolicy);
                    __builtin_amdgcn_raw_buffer_store_b128(f32x4{s[p][4], s[p][5], s[p][6], s[p][7]}, rs,
                                                           voff + kSeg1, p * kPass, kStatePolicy);
                }
            }
        }
    }
    if (tid == 0) s_last = arrived == G - 1;
    __syncthreads();
    if (s_last) {   // the last workgroup of the group rolls the q/k window
        if (commit > 0) {
            for (int e = tid; e < (K - 1) * 2 * D; e += kRowThreads) {
                const int r = e / (2 * D), c = e % (2 * D);
                const int gc = c < D ? g * D + c : P.h_k * D + g * D + (c - D);
                Io<T>::store(win, (int64_t)r * C + gc, line[r * 2 * D + c]);
            }
        }
        if (tid == 0) atomicExch(ctr, 0);
    }
    // ---- outputs: the head's D values per token, 16-byte vectors.
    if (out) {
        constexpr int VN = 16 / sizeof(T);
        for (int e = tid; e < n_tok * (D / VN); e += kRowThreads) {
            const int t = e / (D / VN), j = (e % (D / VN)) * VN;
            const float* src = obuf + t * D + j;
            T* dst = out + (((int64_t)i * n_tok + t) * P.h_v + hv) * D + j;
            if constexpr (sizeof(T) == 2) {
                uint4 uu;
                uu.x = f32_to_bf16(src[0]) | ((uint32_t)f32_to_bf16(src[1]) << 16);
                uu.y = f32_to_bf16(src[2]) | ((uint32_t)f32_to_bf16(src[3]) << 16);
                uu.z = f32_to_bf16(src[4]) | ((uint32_t)f32_to_bf16(src[5]) << 16);
                uu.w = f32_to_bf16(src[6]) | ((uint32_t)f32_to_bf16(src[7]) << 16);
                *reinterpret_cast<uint4*>(dst) = uu;
            } else {
                *reinterpret_cast<float4*>(dst) = make_float4(src[0], src[1], src[2], src[3]);
            }
        }
    }
}

template <int D, typename T, int KC, int NB, bool DECODE>
hipError_t launch_heads_k(const gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                          int32_t n_tok, const void* q, const void* k, const void* v,
                          const float* a, const float* b, const float* conv_w,
                          const int32_t* accept_len, void* out, hipStream_t stream) {
    const PoolView& P = pool->view;
    constexpr int KM = KC > 0 ? KC : kMaxConvK;
    constexpr int NTM = DECODE ? 1 : NB;
    const size_t lds =
        ((size_t)(KM - 1) * 2 * D + (size_t)NTM * 3 * D + 8 * NTM + (size_t)NTM * D) * sizeof(float);
    hipLaunchKernelGGL((decode_heads_kernel<D, T, KC, NB, DECODE>), dim3(P.h_v, n), dim3(kRowThreads),
                       lds, stream, P, layer, slot_ids, n_tok, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), a, b, conv_w, accept_len,
                       static_cast<T*>(out));
    return hipGetLastError();
}

template <int D, typename T, int NB, bool DECODE>
hipError_t launch_heads(const gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                        int32_t n_tok, const void* q, const void* k, const void* v, const float* a,
                        const float* b, const float* conv_w, const int32_t* accept_len, void* out,
                        hipStream_t stream) {
    if (pool->view.conv_k == 4)
        return launch_heads_k<D, T, 4, NB, DECODE>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b,
                                                   conv_w, accept_len, out, stream);
    return launch_heads_k<D, T, 0, NB, DECODE>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b,
                                               conv_w, accept_len, out, stream);
}

template <int D, typename T>
hipError_t launch_heads_n(const gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                          int32_t n_tok, const void* q, const void* k, const void* v,
                          const float* a, const float* b, const float* conv_w,
                          const int32_t* accept_len, void* out, hipStream_t stream) {
    if (n_tok == 1 && !accept_len)
        return launch_heads<D, T, 1, true>(pool, layer, n, slot_ids, 1, q, k, v, a, b, conv_w,
                                           nullptr, out, stream);
    static_assert(kMaxVerifyTokens == 8, "token bounds below cover 1..8");
    if (n_tok <= 2)
        return launch_heads<D, T, 2, false>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                                            accept_len, out, stream);
    if (n_tok <= 4)
        return launch_heads<D, T, 4, false>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                                            accept_len, out, stream);
    return launch_heads<D, T, 8, false>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                                        accept_len, out, stream);
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

bool decode_heads_ok(const gdn_pool* pool) {
    return pool->view.d == 128 || pool->view.d == 64;
}

hipError_t launch_decode_heads(const gdn_pool* pool, int32_t layer, int32_t n,
                               const int32_t* slot_ids, int32_t n_tok, const void* q,
                               const void* k, const void* v, const float* a, const float* b,
                               const float* conv_w, const int32_t* accept_len, void* out,
                               hipStream_t stream) {
    const bool bf = pool->desc.io_dtype == GDN_BF16;
    if (pool->view.d == 128)
        return bf ? launch_heads_n<128, uint16_t>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b,
                                                  conv_w, accept_len, out, stream)
                  : launch_heads_n<128, float>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b,
                                               conv_w, accept_len, out, stream);
    return bf ? launch_heads_n<64, uint16_t>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                                             accept_len, out, stream)
              : launch_heads_n<64, float>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                                          accept_len, out, stream);
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
