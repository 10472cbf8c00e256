// Speculative verify over a ring of committed tokens: outputs now, commit
// after sampling, and a full state write only when the ring fills up
// ("Plan (research-based): Qwen3.6-35B-A3B", section "What the research
// found": output-only ring reconstruction with the chunked (I+A)^-1
// UT-transform, the full state flushed only every L tokens; section "The
// plan", Phase 1: the ring holds at least twice the longest speculation).
//
// A pool built with ring_len = L > 0 keeps, per slot and layer, besides the
// state tile S and the conv window: a count c <= L and the post-conv k^ (per
// q/k head), v (per value head), a and b of the c tokens committed since S
// was last written.  The slot's logical state is S advanced by those c
// tokens; its conv window is always current.
//
// Both kernels solve the c ring tokens followed by up to 8 new tokens as one
// chunk of at most 32 tokens, starting from S, in the UT-transform form:
//     g_t = sum_{s<=t} log a_s,   gamma_t = exp(g_t)
//     A[t][s] = b_t exp(g_t - g_s) k^_t.k^_s   (s < t),   T = (I + A)^-1
//     U  = T diag(b) (V - diag(gamma) K S^T)
//     O  = diag(gamma) Q S^T + P U,   P[t][s] = exp(g_t - g_s) q^_t.k^_s  (s <= t)
//     S' = exp(g_last) S + U^T diag(exp(g_last - g)) K
// ring_verify writes O for the draft rows and writes nothing to the pool.
// ring_commit appends the accepted tokens to the ring; if they do not fit,
// it folds ring + accepted tokens into S (S' above) and empties the ring.
// Either way the conv window advances by the accepted tokens.  A flush is a
// commit of no tokens that folds a non-empty ring.
//
// One workgroup per (entry, value head), four waves; wave w owns state row
// tiles w, w+4 (16 rows of d_v each).  The state is read once, straight into
// MFMA operand registers: lane (m, q) of row tile rt holds row 16 rt + m at
// d_k 32 ks + 4q + i and 32 ks + 16 + 4q + i (i < 4) for each k-step ks.  Read
// as the B operand of K S^T, these are k = 8q..8q+7 in a permuted d_k order
// (the K^ operand uses the same order); read as accumulators, they are
// exactly the result tiles of the state update S'^T = ... + K^T U~.  Token
// contractions use the same device on the token axis: a lane of a 16x16 tile
// result holds tokens 4q..4q+3 of tile 0 and, one tile down, 16+4q.. of
// tile 1, which is one 32-token B operand in permuted order, so results feed
// the next MFMA without any cross-lane move.
#include "gdn_common.h"
#include "mfma_split.h"

namespace gdn {
namespace {

constexpr float kLogDecayMin = -87.f;

// Four waves per workgroup; wave w owns state row tiles w, w + 4, ...  (One
// wave per row tile at d = 128 was measured slower: twice the waves per
// workgroup leave room for two workgroups per CU instead of three, so
// fewer state tiles stream at once.)
constexpr int ring_waves(int) { return 4; }
constexpr int ring_threads(int d) { return 64 * ring_waves(d); }

// Token slots of a permuted 32-token operand: element e of lane quarter q.
__device__ __forceinline__ int tok_slot(int q, int e) { return e < 4 ? 4 * q + e : 16 + 4 * q + e - 4; }

// Buffer descriptors (raw, 32-bit offsets): a load at or past `bytes`
// returns zero without a memory access.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kOffOOB = 0x7fff0000;     // an offset past every descriptor used here
// State tile loads with the default cache policy (the fold's stores are
// non-temporal): measured at 128 slots x 4 drafts, a verify + commit cycle
// took 146 us, against 163 us with non-temporal loads.
constexpr int kStreamPolicy = 0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcWord3);
}
template <int POLICY = 0>
__device__ __forceinline__ f32x4 ld_b128(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY);
}
__device__ __forceinline__ float ld_b32(__amdgpu_buffer_rsrc_t r, int off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

template <typename T>
__device__ __forceinline__ T* window_of(const PoolView& P, int64_t sl) {
    return reinterpret_cast<T*>(P.window) + sl * (int64_t)(P.conv_k - 1) * P.c_conv;
}

enum { kModeVerify = 0, kModeCommit = 1, kModeFlush = 2 };

// acc[j] += a[j] * b[j] for N independent tiles (see mma3_n), with operands
// given by index tables so that tiles can share fragments.
template <int N>
__device__ __forceinline__ void mma3_idx(f32x4* acc, const Frag* const* a, const Frag* const* b) {
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j]->lo, b[j]->hi, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j]->hi, b[j]->lo, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j]->hi, b[j]->hi, acc[j], 0, 0, 0);
}

// MODE: verify (outputs of n_tok draft tokens), commit or flush.  NT = token
// tiles of the solve (ring_len + n_tok <= 16 NT).  KC > 0: conv taps fixed at
// compile time (= conv_k); NTM: most new tokens per call (n_tok <= NTM).
template <int D, int NT, int MODE, int KC, int NTM, typename T>
__device__ __forceinline__ void ring_item(
    PoolView P, int layer, const int32_t* __restrict__ slot_ids, int n_tok,
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, const float* __restrict__ conv_w,
    const int32_t* __restrict__ accept_len, T* __restrict__ out, const int e, const int h) {
    constexpr int NTOK = 16 * NT;          // tokens of the solve (padded)
    constexpr int KP = D + 4;              // row of kn / qn (floats)
    constexpr int MP = NTOK + 4;           // row of vt and of the token matrices
    constexpr int NKS = D / 32;            // k-steps over d_k
    constexpr int RT = D / 16;             // state row tiles
    constexpr int NWAVE = ring_waves(D);
    constexpr int kThreads = 64 * NWAVE;
    constexpr int RTW = (RT + NWAVE - 1) / NWAVE;   // row tiles per wave
    constexpr int KM = KC > 0 ? KC : kMaxConvK;   // taps of the fixed-size conv
    constexpr int KW = KM - 1;             // window slots of the fixed-size conv
    constexpr int XW = KW + NTM;           // window slots, then token slots
    constexpr bool VERIFY = MODE == kModeVerify, FLUSH = MODE == kModeFlush;
    constexpr int NCH = 3 * D;             // conv channels read: q, k, v of this head
    constexpr int CPT = (NCH + kThreads - 1) / kThreads;
    // k^ rows (ring, then new tokens) and, for a verify, the q^ rows of the
    // drafts; a verify reads them only to split them into fragments, which
    // then go over them (fr below)
    __shared__ __align__(16) float kq[NTOK * KP + (VERIFY ? 16 * KP : 0)];
    float* const kn = kq;
    float* const qn = kq + NTOK * KP;
    __shared__ __align__(16) float vt[D * MP];             // v transposed: [d_v][token]
    __shared__ __align__(16) float mA[NTOK * MP];          // A; later A10 T00
    __shared__ __align__(16) float mT[NTOK * MP];          // T = (I+A)^-1
    __shared__ __align__(16) float mP[VERIFY ? 16 * MP : 4];   // P rows of the drafts
    __shared__ __align__(16) float sg[NTOK], sb[NTOK], sla[NTOK];
    // The cumulative log-decay also in fp64, and exp(g_last - g) from it: with
    // a -> 0 (log a down to the clamp) |g| reaches hundreds, where fp32 keeps
    // only ~1e-5 of the differences that the decays are made of.
    __shared__ __align__(16) double sgd[NTOK];
    __shared__ __align__(16) float sge[NTOK];
    // K^ (token tiles) and Q^ (verify) rows split once into MFMA fragments,
    // fragment ks * NKT + tt: shared by the Gram blocks and X = [K; Q] S^T of
    // every wave (lane (m, q): row 16 tt + m, d_k 32 ks + 4q.. and +16..).  A
    // verify keeps them over its k^/q^ rows; a commit still needs its k^
    // rows (the fold, the ring append), so it keeps them apart.
    constexpr int NKT = NT + (VERIFY ? 1 : 0);
    constexpr int NFR = NKS * NKT;
    static_assert(!VERIFY || NFR * kFragVecs * 16 <= (int)sizeof(kq), "fragments fit over the rows");
    __shared__ __align__(16) bf16x8 fr_sep[VERIFY ? 1 : NFR * kFragVecs];
    bf16x8* const fr = VERIFY ? reinterpret_cast<bf16x8*>(kq) : fr_sep;
    __shared__ int s_last;

    // The thread index through an empty asm: a persistent caller runs this
    // body in a loop, and values derived from it would otherwise be hoisted
    // out of the loop and held in registers across the whole body.
    int tid_opaque = threadIdx.x;
    asm volatile("" : "+v"(tid_opaque));
    const int tid = tid_opaque, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m16 = lane & 15, q4 = lane >> 4;
    const int slot = slot_ids[e];
    if (slot < 0) return;
    if (slot >= P.n_slots) {
        if (h == 0 && tid == 0) atomicOr(P.err, kErrSlotRange);
        return;
    }
    const int G = P.h_v / P.h_k, g = h / G, K = KC > 0 ? KC : P.conv_k, C = P.c_conv, L = P.ring_len;
    const int64_t sl = (int64_t)slot * P.n_layers + layer;
    const int hkd = P.h_k * D, hvd = P.h_v * D;
    T* win = window_of<T>(P, sl);

    // ---- Loads that need only the slot: the ring count, and the raw conv
    // inputs of the new tokens (q, k, v channels of this head: window rows,
    // tokens, taps) with a and b.  Raw values only: conversion and masking
    // wait for the data, so they come after every load is issued.  Addresses
    // are clamped into range, so no load sits in a branch.
    const int c_raw = P.ring_cnt[sl];
    const int acc_raw = (!VERIFY && !FLUSH) ? accept_len[e] : 0;
    T rx[CPT][XW];
    float rw[CPT][KM];
    float new_a = 1.f, new_b = 0.f;
    if constexpr (!FLUSH) {   // a flush has no inputs
        const int tmax = n_tok - 1;
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int ch = min(tid + u * kThreads, NCH - 1);
            // 0 q, 1 k, 2 v.  In a commit only the group's first head reads q
            // (it rolls the q window at once); the others read k there instead.
            const int kind0 = ch / D, cc = ch % D;
            const int kind = (!VERIFY && kind0 == 0 && h % G != 0) ? 1 : kind0;
            const int gc = kind == 0 ? g * D + cc : (kind == 1 ? hkd + g * D + cc : 2 * hkd + h * D + cc);
            const T* src = kind == 0 ? q + ((int64_t)e * n_tok * P.h_k + g) * D + cc
                         : kind == 1 ? k + ((int64_t)e * n_tok * P.h_k + g) * D + cc
                                     : v + ((int64_t)e * n_tok * P.h_v + h) * D + cc;
            const int ts = kind == 2 ? hvd : hkd;
#pragma unroll
            for (int j = 0; j < KW; ++j)   // window row j - (KW - (K-1)), clamped
                rx[u][j] = win[(int64_t)max(j - (KW - (K - 1)), 0) * C + gc];
#pragma unroll
            for (int t = 0; t < NTM; ++t) rx[u][KW + t] = src[(int64_t)min(t, tmax) * ts];
#pragma unroll
            for (int m = 0; m < KM; ++m) rw[u][m] = conv_w[(int64_t)gc * K + max(m - (KM - K), 0)];
        }
        const int ta = min(tid, tmax);
        new_a = a[((int64_t)e * n_tok + ta) * P.h_v + h];
        new_b = b[((int64_t)e * n_tok + ta) * P.h_v + h];
    }
    asm volatile("" ::: "memory");   // keep the loads above here, in order

    const int c = min(max(c_raw, 0), L);
    int n_new;
    bool fold;
    if constexpr (VERIFY) {
        n_new = n_tok;
        fold = false;
    } else if constexpr (FLUSH) {
        n_new = 0;
        fold = c > 0;
    } else {
        n_new = min(max(acc_raw, 0), n_tok);
        fold = c + n_new > L;
    }
    if (!VERIFY && n_new == 0 && !fold) return;   // nothing to commit
    // from here on a verify or a commit has at least one new token
    const bool solve = VERIFY || fold;           // uniform over the workgroup
    const int Lc = solve ? c + n_new : 0;        // tokens in the solve (<= NTOK)

    // ---- The ring records and the state tile, through buffer descriptors
    // sized to what this workgroup needs (the c records and the tile when it
    // solves): a load past the end returns zero without a memory access.  The
    // state is issued last, so everything before it can be waited for while
    // the state streams in.
    float* ring = P.ring + sl * P.ring_stride;
    float* rk = ring;                                       // [L][h_k][D]
    float* rv = rk + (int64_t)L * P.h_k * D;                // [L][h_v][D]
    float* ra = rv + (int64_t)L * P.h_v * D;                // [L][h_v]
    float* rb = ra + (int64_t)L * P.h_v;                    // [L][h_v]
    float* S = P.state + (sl * P.h_v + h) * (int64_t)D * D;
    const int cr = solve ? c : 0;                    // ring records this workgroup reads
    const auto rk_rs = buf_rsrc(rk, cr * hkd * 4), rv_rs = buf_rsrc(rv, cr * hvd * 4);
    const auto ra_rs = buf_rsrc(ra, cr * P.h_v * 4), rb_rs = buf_rsrc(rb, cr * P.h_v * 4);
    constexpr int NRV = NTOK * (D / 4);              // 16-byte vectors per record kind
    constexpr int RV = (NRV + kThreads - 1) / kThreads;
    f32x4 rkx[RV], rvx[RV];
#pragma unroll
    for (int i = 0; i < RV; ++i) {
        const int idx = tid + i * kThreads, t = idx / (D / 4), c4 = (idx % (D / 4)) * 4;
        const bool ok = idx < NRV;
        rkx[i] = ld_b128(rk_rs, ok ? ((t * P.h_k + g) * D + c4) * 4 : kOffOOB);
        rvx[i] = ld_b128(rv_rs, ok ? ((t * P.h_v + h) * D + c4) * 4 : kOffOOB);
    }
    const int tr = min(tid, NTOK - 1);
    const float ring_a = ld_b32(ra_rs, (tr * P.h_v + h) * 4), ring_b = ld_b32(rb_rs, (tr * P.h_v + h) * 4);
    // the state tile: lane (m, q) of row tile rt, k-step ks: row 16 rt + m,
    // d_k 32 ks + 4q .. +3 and 32 ks + 16 + 4q .. +3 (read once: non-temporal)
    const auto s_rs = buf_rsrc(S, solve ? D * D * 4 : 0);
    f32x4 s0[RTW][NKS][2];
#pragma unroll
    for (int i = 0; i < RTW; ++i) {
        const int rt = wave + NWAVE * i;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int off = rt < RT ? ((rt * 16 + m16) * D + ks * 32 + q4 * 4) * 4 : kOffOOB;
            s0[i][ks][0] = ld_b128<kStreamPolicy>(s_rs, off);
            s0[i][ks][1] = ld_b128<kStreamPolicy>(s_rs, off + 64);
        }
    }
    asm volatile("" ::: "memory");   // keep every load above here

    // ---- conv + SiLU of the new tokens, one channel per thread and slot.
    // The window is right-aligned in a fixed KW-slot buffer and the taps in a
    // fixed KM-tap filter, so every register index is a compile-time
    // constant.  A commit computes k and v only, and rolls the q and v window
    // rows at once (no other workgroup reads them; the group's last
    // workgroup rolls k, below).  New row p is sequence position n_new + p of
    // [old rows | new tokens].
    if constexpr (!FLUSH) {
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int ch = tid + u * kThreads;
            if (ch >= NCH) continue;
            const int kind = ch / D, cc = ch % D;
            if (VERIFY || kind != 0) {
                float cx[XW], cw[KM];
#pragma unroll
                for (int j = 0; j < XW; ++j) cx[j] = j < KW - (K - 1) ? 0.f : Io<T>::load(&rx[u][j], 0);
#pragma unroll
                for (int m = 0; m < KM; ++m) cw[m] = m < KM - K ? 0.f : rw[u][m];
#pragma unroll
                for (int t = 0; t < NTM; ++t) {
                    if (t < n_new) {
                        float z = 0.f;
#pragma unroll
                        for (int m = 0; m < KM; ++m) z = fmaf(cw[m], cx[t + m], z);
                        const float y = silu(z);
                        if (kind == 0) qn[t * KP + cc] = y;
                        else if (kind == 1) kn[(c + t) * KP + cc] = y;
                        else vt[cc * MP + c + t] = y;
                    }
                }
            }
            if constexpr (!VERIFY) {
                if (kind == 2 || (kind == 0 && h % G == 0)) {
                    const int gc = kind == 0 ? g * D + cc : 2 * hkd + h * D + cc;
#pragma unroll
                    for (int j = 0; j < XW; ++j) {
                        const int pr = j - n_new - (KW - (K - 1));
                        if (pr >= 0 && pr < K - 1) win[(int64_t)pr * C + gc] = rx[u][j];
                    }
                }
            }
        }
    }
    // ---- ring records and zero padding of the solve; decays and betas
    if (solve) {
#pragma unroll
        for (int i = 0; i < RV; ++i) {
            const int idx = tid + i * kThreads, t = idx / (D / 4), c4 = (idx % (D / 4)) * 4;
            if (idx >= NRV || (t >= c && t < Lc)) continue;   // new tokens: written by the conv
            *reinterpret_cast<f32x4*>(kn + t * KP + c4) = rkx[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) vt[(c4 + j) * MP + t] = rvx[i][j];
        }
        if constexpr (VERIFY) {
            for (int idx = tid; idx < 16 * (D / 4); idx += kThreads) {
                const int t = idx / (D / 4), c4 = (idx % (D / 4)) * 4;
                if (t >= n_new) *reinterpret_cast<f32x4*>(qn + t * KP + c4) = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    if (tid < NTOK) {   // raw a for now (the ring stores raw a)
        if (tid < c || tid >= c + n_new) {
            sla[tid] = tid < c && solve ? ring_a : 1.f;
            sb[tid] = tid < c && solve ? ring_b : 0.f;
        }
        if (tid < n_new) {
            sla[c + tid] = new_a;
            sb[c + tid] = new_b;
        }
    }
    __syncthreads();

    // Every read of the slot's conv window and ring count is done: a commit
    // reports its arrival to its q/k group (looked at only at the end).
    int arrived = 0;
    if (!VERIFY && tid == 0) arrived = atomicAdd(P.ctr + sl * P.h_k + g, 1);

    // ---- q/k normalisation of the new tokens (a wave per token), and the
    // cumulative log-decay of the solve
    for (int t = wave; t < n_new; t += NWAVE) {
        float* kr = kn + (c + t) * KP;
        float ss = 0.f;
        for (int j = lane; j < D; j += 64) ss = fmaf(kr[j], kr[j], ss);
        const float rk_ = 1.0f / sqrtf(wave_sum(ss) + P.eps);
        for (int j = lane; j < D; j += 64) kr[j] *= rk_;
        if constexpr (VERIFY) {
            float* qr = qn + t * KP;
            float sq = 0.f;
            for (int j = lane; j < D; j += 64) sq = fmaf(qr[j], qr[j], sq);
            const float rq = P.q_scale / sqrtf(wave_sum(sq) + P.eps);
            for (int j = lane; j < D; j += 64) qr[j] *= rq;
        }
    }
    if (wave == 0 && solve) {
        double la = 0.0;
        if (lane < NTOK) {
            const float av = sla[lane];
            la = lane < Lc ? (double)fmaxf(__logf(av), kLogDecayMin) : 0.0;   // a <= 0 gives -inf -> clamp
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double y = __shfl_up(la, o);
            if (lane >= o) la += y;
        }
        const double gl = __shfl(la, NTOK - 1);   // g is constant past Lc
        if (lane < NTOK) {
            sg[lane] = (float)la;
            sgd[lane] = la;
            sge[lane] = __expf((float)(gl - la));
        }
    }
    __syncthreads();

    if (!solve) {
        // ---- append the accepted tokens to the ring (k^ by the first value
        // head of the group, which all of the group's heads share)
        for (int idx = tid; idx < n_new * (D / 4); idx += kThreads) {
            const int t = idx / (D / 4), c4 = (idx % (D / 4)) * 4;
            if (h % G == 0)
                *reinterpret_cast<float4*>(rk + ((int64_t)(c + t) * P.h_k + g) * D + c4) =
                    *reinterpret_cast<const float4*>(kn + (c + t) * KP + c4);
            *reinterpret_cast<float4*>(rv + ((int64_t)(c + t) * P.h_v + h) * D + c4) =
                make_float4(vt[(c4 + 0) * MP + c + t], vt[(c4 + 1) * MP + c + t],
                            vt[(c4 + 2) * MP + c + t], vt[(c4 + 3) * MP + c + t]);
        }
        if (tid < n_new) {
            ra[(int64_t)(c + tid) * P.h_v + h] = sla[c + tid];
            rb[(int64_t)(c + tid) * P.h_v + h] = sb[c + tid];
        }
    } else {
        // ---- K^ / Q^ fragments, each split once for the workgroup (all rows
        // are read before any fragment is written: they share LDS in a verify)
        constexpr int FPW = (NFR + NWAVE - 1) / NWAVE;
        Frag frw[FPW];
#pragma unroll
        for (int i = 0; i < FPW; ++i) {
            const int f = min(wave + i * NWAVE, NFR - 1);
            const int ks = f / NKT, tt = f % NKT;
            const float* row = (tt < NT ? kn + (tt * 16 + m16) * KP : qn + m16 * KP) + ks * 32 + q4 * 4;
            float x[8];
            ld4x2(x, row, row + 16);
            frw[i] = split8(x);
        }
        if constexpr (VERIFY) __syncthreads();
#pragma unroll
        for (int i = 0; i < FPW; ++i)
            if (wave + i * NWAVE < NFR) store_frag(fr, wave + i * NWAVE, lane, frw[i]);
        __syncthreads();
        // ---- Gram blocks on the matrix cores: KK^T (lower blocks) -> A and
        // QK^T (verify) -> P, with the decays applied on the way to LDS
        constexpr int NKK = NT * (NT + 1) / 2;
        constexpr int NJOB = NKK + (VERIFY ? NT : 0);
        for (int job = wave; job < NJOB; job += NWAVE) {
            const bool isq = job >= NKK;
            const int ti = isq ? 0 : (job == 0 ? 0 : 1), tj = isq ? job - NKK : (job == 2 ? 1 : 0);
            const int fa = isq ? NT : ti, fb = tj;   // fragment tiles of the two operands
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                acc = mma3(acc, load_frag(fr, ks * NKT + fa, lane), load_frag(fr, ks * NKT + fb, lane));
            const int s = tj * 16 + m16;             // column token
            const double gs = sgd[s];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = ti * 16 + q4 * 4 + i;  // row: token (KK) or draft (QK)
                if (!isq) {
                    const float av = s < r ? sb[r] * __expf(fminf((float)(sgd[r] - gs), 0.f)) * acc[i] : 0.f;
                    mA[r * MP + s] = av;
                    if (ti != tj) mA[(tj * 16 + q4 * 4 + i) * MP + ti * 16 + m16] = 0.f;   // upper block
                } else if constexpr (VERIFY) {
                    float pv = 0.f;
                    if (r < n_new) {
                        const int tr2 = c + r;       // the draft's position in the solve
                        pv = s <= tr2 ? __expf(fminf((float)(sgd[tr2] - gs), 0.f)) * acc[i] : 0.f;
                    }
                    mP[r * MP + s] = pv;
                }
            }
        }
        __syncthreads();

        // ---- T = (I + A)^-1: 16x16 diagonal blocks by forward substitution,
        // one wave each (lane = 4 * column + part; part p keeps rows 4p..4p+3
        // of the column), then T10 = -T11 (A10 T00)
        if (wave < NT) {
            const int blk = wave * 16, col = lane >> 2, part = lane & 3;
            float tq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // row r of the block's A (this part's four columns), read at its
                // step: 4 registers instead of 64 beside the state tile
                const float4 a4 = *reinterpret_cast<const float4*>(mA + (blk + r) * MP + blk + 4 * part);
                const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = fmaf(ar[i], tq[i], acc);
                acc = group_sum<4>(acc);
                const float trc = r == col ? 1.f : (r > col ? -acc : 0.f);
#pragma unroll
                for (int i = 0; i < 4; ++i) tq[i] = (4 * part + i == r) ? trc : tq[i];
                if (part == 0) mT[(blk + r) * MP + blk + col] = trc;
            }
        }
        __syncthreads();
        if constexpr (NT == 2) {
            const int r = (tid >> 4) & 15, cl = tid & 15;   // one 16x16 entry per thread
            if (tid < 256) {   // M = A10 T00 into A's upper block
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc = fmaf(mA[(16 + r) * MP + m], mT[m * MP + cl], acc);
                mA[r * MP + 16 + cl] = acc;
            }
            __syncthreads();
            if (tid < 256) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc = fmaf(mT[(16 + r) * MP + 16 + m], mA[m * MP + 16 + cl], acc);
                mT[(16 + r) * MP + cl] = -acc;
                mT[r * MP + 16 + cl] = 0.f;
            }
            __syncthreads();
        }

        // ---- the wave's row tiles together (independent MFMA chains
        // interleaved): X = [K; Q] S^T, R = b (V - gamma X_K), U = T R, then
        // O = gamma X_Q + P U (verify) or S' (fold)
        const float glast = sg[Lc - 1];
        constexpr int NQ = VERIFY ? 1 : 0;
        constexpr int NX = RTW * (NT + NQ);      // X accumulators per wave
        f32x4 xacc[NX];
#pragma unroll
        for (int j = 0; j < NX; ++j) xacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        static_assert(NT + NQ == NKT, "fragment tiles of X");
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            Frag kf[NT + NQ], sf[RTW];
#pragma unroll
            for (int tt = 0; tt < NT + NQ; ++tt) kf[tt] = load_frag(fr, ks * NKT + tt, lane);
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[j] = s0[i][ks][0][j];
                    x[4 + j] = s0[i][ks][1][j];
                }
                sf[i] = split8(x);
            }
            const Frag* fa[NX];
            const Frag* fb[NX];
#pragma unroll
            for (int i = 0; i < RTW; ++i)
#pragma unroll
                for (int tt = 0; tt < NT + NQ; ++tt) {
                    fa[i * (NT + NQ) + tt] = &kf[tt];
                    fb[i * (NT + NQ) + tt] = &sf[i];
                }
            mma3_idx<NX>(xacc, fa, fb);
        }
        // R = b (V - gamma X_K): lane holds tokens 4q+i (tile 0) and 16+4q+i
        // (tile 1) of state row 16 rt + m16, a permuted 32-token B operand
        float4 gq4[NT], bq4[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            gq4[tt] = *reinterpret_cast<const float4*>(sg + tt * 16 + q4 * 4);
            bq4[tt] = *reinterpret_cast<const float4*>(sb + tt * 16 + q4 * 4);
        }
        Frag rf[RTW];
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            const int rt = min(wave + NWAVE * i, RT - 1);
            float rr[8];
            const float* vrow = vt + (rt * 16 + m16) * MP;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                if (tt < NT) {
                    const float4 v4 = *reinterpret_cast<const float4*>(vrow + tt * 16 + q4 * 4);
                    const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
                    const float gg[4] = {gq4[tt].x, gq4[tt].y, gq4[tt].z, gq4[tt].w};
                    const float bb[4] = {bq4[tt].x, bq4[tt].y, bq4[tt].z, bq4[tt].w};
                    const f32x4 xk = xacc[i * (NT + NQ) + tt];
#pragma unroll
                    for (int j = 0; j < 4; ++j) rr[tt * 4 + j] = bb[j] * (vv[j] - __expf(gg[j]) * xk[j]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) rr[tt * 4 + j] = 0.f;
                }
            }
            rf[i] = split8(rr);
        }
        // U = T R: T rows are the A operand, k = 32 tokens in permuted order
        Frag tf[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            float x[8];
            const float* row = mT + (tt * 16 + m16) * MP;
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = (NT == 2 || j < 4) ? row[tok_slot(q4, j)] : 0.f;
            tf[tt] = split8(x);
        }
        constexpr int NU = RTW * NT;
        f32x4 uacc[NU];
        {
            const Frag* fa[NU];
            const Frag* fb[NU];
#pragma unroll
            for (int i = 0; i < RTW; ++i)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    uacc[i * NT + tt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    fa[i * NT + tt] = &tf[tt];
                    fb[i * NT + tt] = &rf[i];
                }
            mma3_idx<NU>(uacc, fa, fb);
        }
        Frag uf[RTW];
#pragma unroll
        for (int i = 0; i < RTW; ++i) {
            float uu[8];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int ts = min(tt, NT - 1);
                const f32x4 u = uacc[i * NT + ts];
                const float4 e4 = *reinterpret_cast<const float4*>(sge + ts * 16 + q4 * 4);
                const float ee[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float x = tt < NT ? u[j] : 0.f;
                    if constexpr (!VERIFY) x *= ee[j];   // decayed U for the state update
                    uu[tt * 4 + j] = x;
                }
            }
            uf[i] = split8(uu);
        }
        if constexpr (VERIFY) {
            // O = gamma X_Q + P U: P rows (drafts) are the A operand
            Frag pf;
            {
                float x[8];
                const float* row = mP + m16 * MP;
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = (NT == 2 || j < 4) ? row[tok_slot(q4, j)] : 0.f;
                pf = split8(x);
            }
            f32x4 oacc[RTW];
            const Frag* fa[RTW];
            const Frag* fb[RTW];
            float gd[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) gd[j] = __expf(sg[min(c + q4 * 4 + j, NTOK - 1)]);
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const f32x4 xq = xacc[i * (NT + NQ) + NT];
                oacc[i] = f32x4{gd[0] * xq[0], gd[1] * xq[1], gd[2] * xq[2], gd[3] * xq[3]};
                fa[i] = &pf;
                fb[i] = &uf[i];
            }
            mma3_idx<RTW>(oacc, fa, fb);
#pragma unroll
            for (int i = 0; i < RTW; ++i) {
                const int rt = wave + NWAVE * i;
                if (rt >= RT) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int td = q4 * 4 + j;
                    if (td < n_new)
                        Io<T>::store(out, (((int64_t)e * n_tok + td) * P.h_v + h) * D + rt * 16 + m16, oacc[i][j]);
                }
            }
        } else {
            // S'^T tile (d_k tile j, row tile) = exp(g_last) S^T + K^T U~: the
            // accumulators start from the state registers and end as the rows
            // to store (lane: row 16 rt + m16, d_k 16 j + 4q .. +3)
            const float dl = __expf(glast);
#pragma unroll
            for (int j = 0; j < D / 16; ++j) {
                float x[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    x[jj] = (NT == 2 || jj < 4) ? kn[tok_slot(q4, jj) * KP + j * 16 + m16] : 0.f;
                const Frag kf = split8(x);
                f32x4 sacc[RTW];
                const Frag* fa[RTW];
                const Frag* fb[RTW];
#pragma unroll
                for (int i = 0; i < RTW; ++i) {
                    sacc[i] = dl * s0[i][j / 2][j % 2];
                    fa[i] = &kf;
                    fb[i] = &uf[i];
                }
                mma3_idx<RTW>(sacc, fa, fb);
#pragma unroll
                for (int i = 0; i < RTW; ++i) {
                    const int rt = wave + NWAVE * i;
                    if (rt >= RT) continue;
                    __builtin_nontemporal_store(sacc[i], reinterpret_cast<f32x4*>(S + (int64_t)(rt * 16 + m16) * D + j * 16 + q4 * 4));
                }
            }
        }
    }

    if constexpr (!VERIFY) {
        // ---- The k window channels are read by every value head of the
        // group: the group's last workgroup to arrive rolls them (from the
        // values it loaded), and the slot's last group sets the ring count
        // (every workgroup read the count before arriving).  Counters return
        // to zero.
        if (tid == 0) {
            int flag = 0;
            if (arrived == G - 1) {
                flag = 1;
                atomicExch(P.ctr + sl * P.h_k + g, 0);
                if (atomicAdd(P.ring_arr + sl, 1) == P.h_k - 1) {
                    P.ring_cnt[sl] = fold ? 0 : c + n_new;
                    atomicExch(P.ring_arr + sl, 0);
                }
            }
            s_last = flag;
        }
        __syncthreads();
        if constexpr (!FLUSH) {
            if (s_last) {
#pragma unroll
                for (int u = 0; u < CPT; ++u) {
                    const int ch = tid + u * kThreads;
                    if (ch >= NCH || ch / D != 1) continue;
                    const int gc = hkd + g * D + ch % D;
#pragma unroll
                    for (int j = 0; j < XW; ++j) {
                        const int pr = j - n_new - (KW - (K - 1));
                        if (pr >= 0 && pr < K - 1) win[(int64_t)pr * C + gc] = rx[u][j];
                    }
                }
            }
        }
    }
}

// Most entries a persistent commit orders (fold-first) in LDS.
constexpr int kRingPersistMax = 1024;

// One workgroup per (entry, value head), or, for a commit with persist != 0,
// a persistent grid of one round of workgroups walking the (entry, head)
// items with a stride of the grid: folding entries first (a fold solves and
// writes the state, ~3x an append's time), so that the long items start
// early and the appends fill in behind them, with no workgroup dispatched
// per short append.  The order is a stable partition of the entries by the
// fold test the item itself makes (ring count + accepted tokens > L).
template <int D, int NT, int MODE, int KC, int NTM, typename T>
// A verify with one token tile and a fixed conv width (the common shape)
// runs four workgroups per CU: 120 VGPRs without spills, and four state tiles
// streaming per CU instead of three.
__global__ __launch_bounds__(ring_threads(D), MODE == kModeVerify && NT == 1 && KC > 0 ? 4 : 1) void ring_kernel(
    PoolView P, int layer, const int32_t* __restrict__ slot_ids, int n_tok,
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, const float* __restrict__ conv_w,
    const int32_t* __restrict__ accept_len, T* __restrict__ out) {
    ring_item<D, NT, MODE, KC, NTM, T>(P, layer, slot_ids, n_tok, q, k, v, a, b, conv_w, accept_len,
                                       out, blockIdx.x, blockIdx.y);
}

template <int D, int NT, int KC, int NTM, typename T>
__global__ __launch_bounds__(ring_threads(D), 3) void ring_commit_persistent_kernel(
    PoolView P, int layer, const int32_t* __restrict__ slot_ids, int n_tok,
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ a, const float* __restrict__ b, const float* __restrict__ conv_w,
    const int32_t* __restrict__ accept_len, int n) {
    constexpr int MODE = kModeCommit;
    {
        {
            __shared__ int s_ord[kRingPersistMax];
            const int tid = threadIdx.x, lane = tid & 63;
            if (tid < 64) {   // wave 0: lane l takes entries [l*per, (l+1)*per)
                const int per = (n + 63) / 64, e0 = min(lane * per, n), e1 = min(e0 + per, n);
                const auto folds = [&](int e) {
                    const int slot = slot_ids[e];
                    if (slot < 0 || slot >= P.n_slots) return false;
                    const int c = min(max(P.ring_cnt[(int64_t)slot * P.n_layers + layer], 0), P.ring_len);
                    return c + min(max(accept_len[e], 0), n_tok) > P.ring_len;
                };
                int nf = 0;
                for (int e = e0; e < e1; ++e) nf += folds(e);
                int incl = nf;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(incl, o);
                    if (lane >= o) incl += y;
                }
                const int total_f = __shfl(incl, 63);
                int pf = incl - nf, pa = total_f + (e0 - (incl - nf));   // first fold / append slot
                for (int e = e0; e < e1; ++e) {
                    if (folds(e)) s_ord[pf++] = e;
                    else s_ord[pa++] = e;
                }
            }
            __syncthreads();
#pragma unroll 1
            for (int i = blockIdx.x; i < n * P.h_v; i += gridDim.x) {
                // (the entry through readfirstlane: known uniform, so its addresses stay scalar)
                ring_item<D, NT, MODE, KC, NTM, T>(P, layer, slot_ids, n_tok, q, k, v, a, b, conv_w,
                                                   accept_len, nullptr,
                                                   __builtin_amdgcn_readfirstlane(s_ord[i / P.h_v]),
                                                   i % P.h_v);
                __syncthreads();
            }
        }
    }
}

template <int D, int NT, int MODE, int KC, int NTM, typename T>
void launch_one(const gdn_pool* pool, int32_t layer, int32_t n, const int32_t* slot_ids,
                int32_t n_tok, const void* q, const void* k, const void* v, const float* a,
                const float* b, const float* conv_w, const int32_t* accept_len, void* out,
                hipStream_t stream) {
    auto kern = ring_kernel<D, NT, MODE, KC, NTM, T>;
    auto pkern = ring_commit_persistent_kernel<D, NT, KC, NTM, T>;
    // A commit runs persistent (one round of workgroups, fold-first order)
    // when its entries fit the order buffer.
    int grid = 0;
    if (MODE == kModeCommit && n <= kRingPersistMax) {
        static std::atomic<int> per_cu{-1};
        int pc = per_cu.load(std::memory_order_relaxed);
        if (pc < 0) {
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, reinterpret_cast<const void*>(pkern),
                                                             ring_threads(D), 0) != hipSuccess)
                pc = 0;
            per_cu.store(pc, std::memory_order_relaxed);
        }
        const int64_t items = (int64_t)n * pool->view.h_v;
        if (pc > 0 && device_cus() > 0 && items > (int64_t)pc * device_cus())
            grid = pc * device_cus();
    }
    if (grid > 0)
        hipLaunchKernelGGL(pkern, dim3(grid), dim3(ring_threads(D)), 0, stream, pool->view, layer,
                           slot_ids, n_tok, static_cast<const T*>(q), static_cast<const T*>(k),
                           static_cast<const T*>(v), a, b, conv_w, accept_len, n);
    else
        hipLaunchKernelGGL(kern, dim3(n, pool->view.h_v), dim3(ring_threads(D)), 0, stream,
                           pool->view, layer, slot_ids, n_tok, static_cast<const T*>(q),
                           static_cast<const T*>(k), static_cast<const T*>(v), a, b, conv_w,
                           accept_len, static_cast<T*>(out));
}

// Compile-time shapes: conv_k = 4 with at most 4 new tokens (the common
// speculation depth) gets its own instance with fewer conv loads.
template <int D, int NT, int MODE, typename T>
void launch_conv(bool fast, const gdn_pool* pool, int32_t layer, int32_t n,
                 const int32_t* slot_ids, int32_t n_tok, const void* q, const void* k,
                 const void* v, const float* a, const float* b, const float* conv_w,
                 const int32_t* accept_len, void* out, hipStream_t stream) {
    if (fast)
        launch_one<D, NT, MODE, 4, 4, T>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                                         accept_len, out, stream);
    else
        launch_one<D, NT, MODE, 0, kMaxVerifyTokens, T>(pool, layer, n, slot_ids, n_tok, q, k, v,
                                                        a, b, conv_w, accept_len, out, stream);
}

template <int D, int NT, typename T>
void launch_mode(int mode, bool fast, const gdn_pool* pool, int32_t layer, int32_t n,
                 const int32_t* slot_ids, int32_t n_tok, const void* q, const void* k,
                 const void* v, const float* a, const float* b, const float* conv_w,
                 const int32_t* accept_len, void* out, hipStream_t stream) {
    if (mode == kModeVerify)
        launch_conv<D, NT, kModeVerify, T>(fast, pool, layer, n, slot_ids, n_tok, q, k, v, a, b,
                                           conv_w, accept_len, out, stream);
    else if (mode == kModeCommit)
        launch_conv<D, NT, kModeCommit, T>(fast, pool, layer, n, slot_ids, n_tok, q, k, v, a, b,
                                           conv_w, accept_len, out, stream);
    else   // a flush reads no conv inputs: one instance
        launch_one<D, NT, kModeFlush, 4, 4, T>(pool, layer, n, slot_ids, n_tok, q, k, v, a, b,
                                               conv_w, accept_len, out, stream);
}

template <int D, typename T>
void launch_nt(int nt, int mode, bool fast, const gdn_pool* pool, int32_t layer, int32_t n,
               const int32_t* slot_ids, int32_t n_tok, const void* q, const void* k,
               const void* v, const float* a, const float* b, const float* conv_w,
               const int32_t* accept_len, void* out, hipStream_t stream) {
    if (nt == 1)
        launch_mode<D, 1, T>(mode, fast, pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                             accept_len, out, stream);
    else
        launch_mode<D, 2, T>(mode, fast, pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                             accept_len, out, stream);
}

template <typename T>
hipError_t launch_d(int nt, int mode, bool fast, const gdn_pool* pool, int32_t layer, int32_t n,
                    const int32_t* slot_ids, int32_t n_tok, const void* q, const void* k,
                    const void* v, const float* a, const float* b, const float* conv_w,
                    const int32_t* accept_len, void* out, hipStream_t stream) {
    switch (pool->view.d) {
        case 32: launch_nt<32, T>(nt, mode, fast, pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w, accept_len, out, stream); break;
        case 64: launch_nt<64, T>(nt, mode, fast, pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w, accept_len, out, stream); break;
        case 128: launch_nt<128, T>(nt, mode, fast, pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w, accept_len, out, stream); break;
        default: return hipErrorNotSupported;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ring(const gdn_pool* pool, RingOp op, int32_t layer, int32_t n,
                       const int32_t* slot_ids, int32_t n_tok, const void* q, const void* k,
                       const void* v, const float* a, const float* b, const float* conv_w,
                       const int32_t* accept_len, void* out, hipStream_t stream) {
    // The solve holds the ring plus the call's tokens: one token tile when
    // they fit in 16, else two (ring_len + n_tok <= 32 is checked by the caller).
    const int nt = pool->view.ring_len + n_tok <= 16 ? 1 : 2;
    const int mode = op == RingOp::kVerify ? kModeVerify : (op == RingOp::kCommit ? kModeCommit : kModeFlush);
    const bool fast = pool->view.conv_k == 4 && n_tok <= 4;
    if (pool->desc.io_dtype == GDN_BF16)
        return launch_d<uint16_t>(nt, mode, fast, pool, layer, n, slot_ids, n_tok, q, k, v, a, b,
                                  conv_w, accept_len, out, stream);
    return launch_d<float>(nt, mode, fast, pool, layer, n, slot_ids, n_tok, q, k, v, a, b, conv_w,
                           accept_len, out, stream);
}

}  // namespace gdn
