// Chunked prefill of packed variable-length sequences into pool slots.
//
// Each sequence is cut into chunks of C tokens aligned to its start; a chunk
// is solved in the UT-transform form of the gated delta rule and the state is
// carried chunk to chunk ("Plan (research-based): Qwen3.6-35B-A3B", "What the
// research found": chunked delta rule with (I+A)^-1; "Project: adding the
// hybrid model Qwen3.5", "What to do", row "State": chunked prefill passes the
// state on).  With g the cumulative log-decay inside a chunk, gamma = exp(g),
// and S0 the state entering the chunk (per value head, [d_v][d_k]):
//     A[t][s] = b_t exp(g_t - g_s) k_t.k_s   (s < t)
//     T'      = (I + A)^-1 diag(b)
//     U       = T' (V - diag(gamma) K S0^T)            new values
//     O       = diag(gamma) Q S0^T + P U,  P[t][s] = exp(g_t - g_s) q_t.k_s (s <= t)
//     S       = exp(g_last) S0 + U^T diag(exp(g_last - g)) K
//
// Three kernels, stream-ordered, no host synchronisation:
//   prep   (1 workgroup)            chunk map from the device cu_seqlens;
//   factor (chunk x q/k head)        conv+SiLU, q/k normalisation, KK^T and QK^T
//                                    on bf16 MFMA, T' and P per value head;
//   scan   (row block x v head x seq) the serial chunk carry: X = [Q;K] S0^T,
//                                    U, O and the state update on bf16 MFMA,
//                                    the state block kept in registers.
// Every MFMA operand that is not an exact bf16 value is split as hi + lo
// bf16 and multiplied as hi*hi + hi*lo + lo*hi (fp32 accumulate), which keeps
// the chunked result within fp32-recurrence accuracy.
#include "gdn_common.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRows = 16;          // state rows (d_v) per scan workgroup
constexpr float kLogDecayMin = -87.f;

// ------------------------------------------------------------ MFMA helpers

struct Split8 {
    bf16x8 hi, lo;
};

__device__ __forceinline__ Split8 split8(const float* x) {
    Split8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 h = (__bf16)x[j];
        r.hi[j] = h;
        r.lo[j] = (__bf16)(x[j] - (float)h);
    }
    return r;
}

// acc += A * B for one 16x16x32 tile, operands split in hi/lo bf16.
__device__ __forceinline__ f32x4 mma3(f32x4 acc, const Split8& a, const Split8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ void ld8(float* dst, const float* src) {
    const float4 x0 = *reinterpret_cast<const float4*>(src);
    const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
    dst[0] = x0.x; dst[1] = x0.y; dst[2] = x0.z; dst[3] = x0.w;
    dst[4] = x1.x; dst[5] = x1.y; dst[6] = x1.z; dst[7] = x1.w;
}

// --------------------------------------------------------------- workspace

struct Ws {
    int32_t* hdr;        // [0]: number of chunks, or -1 if cu_seqlens is malformed
    int32_t* seq_coff;   // [n_seq+1] first global chunk of each sequence
    int32_t* chunk_seq;  // [max_chunks] sequence owning each chunk
    float* qh;           // [max_chunks][h_k][CP][D] normalised, scaled q
    float* kh;           // [max_chunks][h_k][CP][D] normalised k
    float* tq;           // [max_chunks][h_v][CP][CP] T' = (I+A)^-1 diag(b)
    float* pm;           // [max_chunks][h_v][CP][CP] P (lower triangle incl. diagonal)
    float* gl;           // [max_chunks][h_v][CP] cumulative log-decay in the chunk
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int64_t max_chunks(int32_t n_seq, int64_t total, int32_t chunk) {
    return (total + chunk - 1) / chunk + n_seq;
}

int padded_chunk(int32_t chunk) { return chunk < 32 ? 32 : chunk; }

Ws carve(void* base, const PoolView& P, int32_t n_seq, int64_t total, int32_t chunk,
         size_t* bytes) {
    const int64_t mc = max_chunks(n_seq, total, chunk);
    const int64_t CP = padded_chunk(chunk);
    size_t off = 0;
    auto take = [&](size_t n) {
        const size_t o = off;
        off += align256(n);
        return o;
    };
    const size_t o_hdr = take(256);
    const size_t o_coff = take((size_t)(n_seq + 1) * 4);
    const size_t o_cseq = take((size_t)mc * 4);
    const size_t o_q = take((size_t)mc * P.h_k * CP * P.d * 4);
    const size_t o_k = take((size_t)mc * P.h_k * CP * P.d * 4);
    const size_t o_t = take((size_t)mc * P.h_v * CP * CP * 4);
    const size_t o_p = take((size_t)mc * P.h_v * CP * CP * 4);
    const size_t o_g = take((size_t)mc * P.h_v * CP * 4);
    *bytes = off;
    char* b = static_cast<char*>(base);
    Ws w;
    w.hdr = reinterpret_cast<int32_t*>(b + o_hdr);
    w.seq_coff = reinterpret_cast<int32_t*>(b + o_coff);
    w.chunk_seq = reinterpret_cast<int32_t*>(b + o_cseq);
    w.qh = reinterpret_cast<float*>(b + o_q);
    w.kh = reinterpret_cast<float*>(b + o_k);
    w.tq = reinterpret_cast<float*>(b + o_t);
    w.pm = reinterpret_cast<float*>(b + o_p);
    w.gl = reinterpret_cast<float*>(b + o_g);
    return w;
}

// ------------------------------------------------------------------- prep

// One workgroup: check cu_seqlens, count chunks per sequence, prefix-sum them
// and record which sequence owns each chunk.  A malformed cu_seqlens marks
// the workspace invalid (the other kernels then do nothing) and sets the
// sticky error bit.
constexpr int kPrepThreads = 1024;

__global__ __launch_bounds__(kPrepThreads) void prefill_prep_kernel(
    PoolView P, Ws W, const int32_t* __restrict__ cu, int n_seq, int total, int chunk,
    int max_chunks) {
    __shared__ int part[kPrepThreads];
    __shared__ int bad;
    const int tid = threadIdx.x;
    if (tid == 0) bad = 0;
    __syncthreads();
    // Contiguous range of sequences per thread.
    const int per = (n_seq + kPrepThreads - 1) / kPrepThreads;
    const int j0 = min(tid * per, n_seq), j1 = min(j0 + per, n_seq);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) {
        const int s = cu[j], e = cu[j + 1];
        if (s < 0 || e < s || e > total) bad = 1;
        else cnt += (e - s + chunk - 1) / chunk;
    }
    if (tid == 0 && (cu[0] != 0 || cu[n_seq] != total)) bad = 1;
    part[tid] = cnt;
    __syncthreads();
    // Inclusive scan of the per-thread counts (Hillis-Steele).
    for (int o = 1; o < kPrepThreads; o <<= 1) {
        const int x = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += x;
        __syncthreads();
    }
    const int n_chunks = part[kPrepThreads - 1];
    if (bad || n_chunks > max_chunks) {
        if (tid == 0) {
            W.hdr[0] = -1;
            atomicOr(P.err, kErrSeqlens);
        }
        return;
    }
    int c = part[tid] - cnt;  // exclusive prefix
    for (int j = j0; j < j1; ++j) {
        W.seq_coff[j] = c;
        const int n = (cu[j + 1] - cu[j] + chunk - 1) / chunk;
        for (int q = 0; q < n; ++q) W.chunk_seq[c + q] = j;
        c += n;
    }
    if (tid == 0) {
        W.seq_coff[n_seq] = n_chunks;
        W.hdr[0] = n_chunks;
    }
}

// ------------------------------------------------------------- conv helper

// Raw input of channel `gc` at token position p of a sequence starting at
// `s0`: from the input tensor for p >= s0, else from the slot's window
// (window row conv_k-1 + (p - s0)).
template <typename T>
__device__ __forceinline__ float raw_at(const T* src, int64_t stride, const T* win, int C, int K,
                                        int gc, int64_t p, int64_t s0) {
    if (p >= s0) return Io<T>::load(src, p * stride);
    return Io<T>::load(win, (int64_t)(K - 1 + (p - s0)) * C + gc);
}

// ------------------------------------------------------------------ factor

// grid (max_chunks, h_k), 256 threads.  LDS: q^ and k^ [CP][D+4] fp32, then
// reused for A [CP][CP+1] and T [CP][CP+1]; small per-token arrays.
template <int D, int CP, typename T>
__global__ __launch_bounds__(kThreads) void prefill_factor_kernel(
    PoolView P, Ws W, int layer, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ slot_ids, int chunk, const T* __restrict__ q,
    const T* __restrict__ k, const float* __restrict__ a, const float* __restrict__ b,
    const float* __restrict__ conv_w) {
    constexpr int LD = D + 4;          // padded row (floats)
    constexpr int LT = CP + 1;
    constexpr int NT = CP / 16;        // token tiles
    constexpr int NKD = D / 32;        // k-steps over d_k
    extern __shared__ __align__(16) float smem[];
    float* xq = smem;                  // [CP][LD]
    float* xk = xq + CP * LD;          // [CP][LD]
    float* sA = smem;                  // [CP][LT]  (after q^, k^ are consumed)
    float* sT = sA + CP * LT;          // [CP][LT]
    __shared__ float s_rq[CP], s_rk[CP], s_g[CP], s_b[CP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ci = blockIdx.x, g = blockIdx.y;
    const int n_chunks = W.hdr[0];
    if (ci >= n_chunks) return;        // also when the workspace is invalid (-1)
    const int j = W.chunk_seq[ci];
    const int slot = slot_ids[j];
    if (slot < 0 || slot >= P.n_slots) return;
    const int64_t s0 = cu[j];
    const int len = cu[j + 1] - (int)s0;
    const int cpos = ci - W.seq_coff[j];          // chunk index inside the sequence
    const int64_t t0 = s0 + (int64_t)cpos * chunk;
    const int L = min(chunk, len - cpos * chunk); // valid tokens in this chunk
    const int K = P.conv_k, C = P.c_conv, G = P.h_v / P.h_k;
    T* win = reinterpret_cast<T*>(P.window) + ((int64_t)slot * P.n_layers + layer) * (int64_t)(K - 1) * C;

    // ---- conv + SiLU of the q and k channels of head g (one channel per thread).
    for (int c = tid; c < 2 * D; c += kThreads) {
        const bool isk = c >= D;
        const int cc = isk ? c - D : c;
        const int gc = (isk ? P.h_k * D : 0) + g * D + cc;
        const T* src = (isk ? k : q) + (int64_t)g * D + cc;
        const int64_t stride = (int64_t)P.h_k * D;
        float w[kMaxConvK], prev[kMaxConvK - 1];
#pragma unroll
        for (int m = 0; m < kMaxConvK; ++m) w[m] = m < K ? conv_w[(int64_t)gc * K + m] : 0.f;
#pragma unroll
        for (int m = 0; m < kMaxConvK - 1; ++m)
            prev[m] = m < K - 1 ? raw_at(src, stride, win, C, K, gc, t0 - (K - 1) + m, s0) : 0.f;
        float* dst = isk ? xk : xq;
        for (int t = 0; t < CP; ++t) {
            float y = 0.f;
            if (t < L) {
                const float x = Io<T>::load(src, (t0 + t) * stride);
                float z = 0.f;
#pragma unroll
                for (int m = 0; m < kMaxConvK - 1; ++m)
                    if (m < K - 1) z = fmaf(w[m], prev[m], z);
                z = fmaf(w[K - 1], x, z);
                y = silu(z);
#pragma unroll
                for (int m = 0; m < kMaxConvK - 1; ++m)
                    prev[m] = (m == K - 2) ? x : (m < K - 2 ? prev[m + 1] : prev[m]);
            }
            dst[t * LD + cc] = y;
        }
        // The sequence's first chunk owns the window of these channels: after
        // its own reads, store the last conv_k-1 raw inputs of the sequence.
        if (cpos == 0) {
            float nw[kMaxConvK - 1];
#pragma unroll
            for (int m = 0; m < kMaxConvK - 1; ++m)
                nw[m] = m < K - 1 ? raw_at(src, stride, win, C, K, gc, s0 + len - (K - 1) + m, s0) : 0.f;
#pragma unroll
            for (int m = 0; m < kMaxConvK - 1; ++m)
                if (m < K - 1) Io<T>::store(win, (int64_t)m * C + gc, nw[m]);
        }
    }
    __syncthreads();

    // ---- per-token q/k norms (one wave per token).
    for (int t = wave; t < CP; t += kThreads / 64) {
        float sq = 0.f, sk = 0.f;
        for (int c = lane; c < D; c += 64) {
            const float x = xq[t * LD + c], y = xk[t * LD + c];
            sq = fmaf(x, x, sq);
            sk = fmaf(y, y, sk);
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        if (lane == 0) {
            s_rq[t] = P.q_scale / sqrtf(sq + P.eps);
            s_rk[t] = 1.0f / sqrtf(sk + P.eps);
        }
    }
    __syncthreads();
    // Scale in place and store q^, k^ to the workspace.
    {
        float* gq = W.qh + ((int64_t)ci * P.h_k + g) * CP * D;
        float* gk = W.kh + ((int64_t)ci * P.h_k + g) * CP * D;
        for (int e = tid; e < CP * D / 4; e += kThreads) {
            const int t = e / (D / 4), c = (e % (D / 4)) * 4;
            float4 x = *reinterpret_cast<float4*>(xq + t * LD + c);
            float4 y = *reinterpret_cast<float4*>(xk + t * LD + c);
            const float rq = s_rq[t], rk = s_rk[t];
            x.x *= rq; x.y *= rq; x.z *= rq; x.w *= rq;
            y.x *= rk; y.y *= rk; y.z *= rk; y.w *= rk;
            *reinterpret_cast<float4*>(xq + t * LD + c) = x;
            *reinterpret_cast<float4*>(xk + t * LD + c) = y;
            *reinterpret_cast<float4*>(gq + t * D + c) = x;
            *reinterpret_cast<float4*>(gk + t * D + c) = y;
        }
    }
    __syncthreads();

    // ---- KK^T and QK^T lower-triangular tiles: wave w takes tile row w (and
    // w+4 when CP/16 > 4 is not possible here: NT <= 4).  Tile (i, jt), jt <= i.
    const int m16 = lane & 15, q4 = lane >> 4;
    f32x4 kk[NT], qk[NT];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
        kk[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        qk[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int ti = wave;  // tile row
    if (ti < NT) {
#pragma unroll
        for (int ks = 0; ks < NKD; ++ks) {
            float x[8];
            ld8(x, xk + (ti * 16 + m16) * LD + ks * 32 + q4 * 8);
            const Split8 ak = split8(x);
            ld8(x, xq + (ti * 16 + m16) * LD + ks * 32 + q4 * 8);
            const Split8 aq = split8(x);
#pragma unroll
            for (int jt = 0; jt < NT; ++jt) {
                if (jt <= ti) {
                    ld8(x, xk + (jt * 16 + m16) * LD + ks * 32 + q4 * 8);
                    const Split8 bk = split8(x);
                    kk[jt] = mma3(kk[jt], ak, bk);
                    qk[jt] = mma3(qk[jt], aq, bk);
                }
            }
        }
    }
    __syncthreads();   // q^, k^ LDS region is reused below

    // ---- per value head of the group: decay, A, T = (I+A)^-1, T', P.
    for (int hl = 0; hl < G; ++hl) {
        const int hv = g * G + hl;
        // cumulative log-decay and b for the chunk's tokens (zero past L)
        if (wave == 0) {
            float la = 0.f, bt = 0.f;
            if (lane < CP && lane < L) {
                const int64_t tok = t0 + lane;
                la = fmaxf(__logf(a[tok * P.h_v + hv]), kLogDecayMin);
                bt = b[tok * P.h_v + hv];
            }
            // inclusive prefix sum over the wave (CP <= 64)
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(la, o);
                if (lane >= o) la += y;
            }
            if (lane < CP) {
                s_g[lane] = la;
                s_b[lane] = bt;
            }
        }
        __syncthreads();
        // A (strictly lower) into LDS, P to the workspace.
        float* gp = W.pm + ((int64_t)ci * P.h_v + hv) * CP * CP;
        if (ti < NT) {
#pragma unroll
            for (int jt = 0; jt < NT; ++jt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = ti * 16 + q4 * 4 + r;   // row (query / later token)
                    const int s = jt * 16 + m16;          // column
                    float av = 0.f, pv = 0.f;
                    if (jt <= ti && s <= t) {
                        const float dec = __expf(s_g[t] - s_g[s]);
                        pv = qk[jt][r] * dec;
                        if (s < t) av = s_b[t] * dec * kk[jt][r];
                    }
                    sA[t * LT + s] = av;
                    gp[t * CP + s] = pv;
                }
            }
        }
        // Tiles of A above the diagonal band are zero.
        for (int e = tid; e < CP * CP; e += kThreads) {
            const int t = e / CP, s = e % CP;
            if (s / 16 > t / 16) {
                sA[t * LT + s] = 0.f;
                gp[t * CP + s] = 0.f;
            }
        }
        __syncthreads();

        // (I+A)^-1, blocked by 16: diagonal blocks by forward substitution (one
        // wave per block; lane = column * 4 + part, parts split the inner sum),
        // then off-diagonal blocks T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj.
        if (wave < NT) {
            const int blk = wave * 16;
            const int col = lane >> 2, part = lane & 3;
            float tcol[16];   // T[blk+r][blk+col] for the rows done so far
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    if (m < r && (m & 3) == part && m >= col)
                        acc = fmaf(sA[(blk + r) * LT + blk + m], tcol[m], acc);
                acc = group_sum<4>(acc);
                tcol[r] = (r == col) ? 1.f : (r > col ? -acc : 0.f);
                if (part == 0) sT[(blk + r) * LT + blk + col] = tcol[r];
            }
        }
        __syncthreads();
        for (int dist = 1; dist < NT; ++dist) {
            // blocks (i, i-dist); 256 threads cover (NT-dist) blocks of 256 entries
            for (int e = tid; e < (NT - dist) * 256; e += kThreads) {
                const int bi = e / 256 + dist, bj = bi - dist;
                const int r = (e % 256) / 16, c = e % 16;
                // M = sum_{m=bj}^{bi-1} A[bi][m] T[m][bj]  (row r, col c), then -T_ii M
                float acc = 0.f;
                for (int mb = bj; mb < bi; ++mb)
                    for (int x = 0; x < 16; ++x)
                        acc = fmaf(sA[(bi * 16 + r) * LT + mb * 16 + x],
                                   sT[(mb * 16 + x) * LT + bj * 16 + c], acc);
                // stash M in the (still zero) upper block (bj, bi) of A
                sA[(bj * 16 + r) * LT + bi * 16 + c] = acc;
            }
            __syncthreads();
            for (int e = tid; e < (NT - dist) * 256; e += kThreads) {
                const int bi = e / 256 + dist, bj = bi - dist;
                const int r = (e % 256) / 16, c = e % 16;
                float acc = 0.f;
                for (int x = 0; x < 16; ++x)
                    acc = fmaf(sT[(bi * 16 + r) * LT + bi * 16 + x], sA[(bj * 16 + x) * LT + bi * 16 + c], acc);
                sT[(bi * 16 + r) * LT + bj * 16 + c] = -acc;
            }
            __syncthreads();
        }
        // T' = T diag(b), upper part zero; write to the workspace.
        float* gt = W.tq + ((int64_t)ci * P.h_v + hv) * CP * CP;
        for (int e = tid; e < CP * CP; e += kThreads) {
            const int t = e / CP, s = e % CP;
            gt[e] = (s <= t) ? sT[t * LT + s] * s_b[s] : 0.f;
        }
        if (tid < CP) W.gl[((int64_t)ci * P.h_v + hv) * CP + tid] = s_g[tid];
        __syncthreads();
    }
}

// -------------------------------------------------------------------- scan

// grid: one workgroup per (sequence, value head, block of 16 state rows), 256 threads.  Wave w < D/32 owns the
// state tiles 2w, 2w+1 of S^T (d_k x rows) for rows rb*16.. of value head h,
// in MFMA accumulator layout: lane l holds S[row l%16][16 tile + 4 (l/16) + i].
// The same registers, read as k-slots {32w+4q+i, 32w+16+4q+i} (q = l/16), are
// the B operand of [Q;K] S^T for k-step w; Q and K fragments are loaded with
// that d_k order.
template <int D, int CP, typename T>
__global__ __launch_bounds__(kThreads) void prefill_scan_kernel(
    PoolView P, Ws W, int layer, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ slot_ids, int chunk, const T* __restrict__ v,
    const float* __restrict__ conv_w, T* __restrict__ out) {
    constexpr int NKS = D / 32;       // d_k slices = waves owning state
    constexpr int NT = CP / 16;       // token tiles
    constexpr int NM = 2 * NT;        // M tiles of [Q;K]
    constexpr int LR = CP + 4;        // padded row of transposed [rows][tokens] tiles
    __shared__ __align__(16) float s_v[CP][kRows];            // conv+SiLU of v for the block
    __shared__ __align__(16) float s_xp[NKS][NM][256];        // partial [Q;K] S^T per d_k slice
    __shared__ __align__(16) float s_rt[kRows][LR];           // R^T
    __shared__ __align__(16) float s_ut[kRows][LR];           // U^T
    __shared__ __align__(16) float s_uu[kRows][LR];           // (diag(exp(g_last - g)) U)^T
    __shared__ __align__(16) float s_xq[CP][kRows];           // diag(gamma) Q S0^T
    __shared__ float s_win[kMaxConvK - 1][kRows];
    __shared__ float s_g[CP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m16 = lane & 15, q4 = lane >> 4;
    // Work unit u = (seq * h_v + h) * (D/16) + rb.  Consecutive workgroup ids
    // go to different XCDs (round robin over 8); when the unit count allows,
    // give each XCD a contiguous range of units so the row blocks of one head
    // (which read the same chunk operands) share that XCD's L2.
    constexpr int NRB = D / kRows;
    const int n_units = gridDim.x;
    const int b = blockIdx.x;
    const int u = (n_units % 8 == 0) ? (b % 8) * (n_units / 8) + b / 8 : b;
    const int rb = u % NRB, h = (u / NRB) % P.h_v, j = u / (NRB * P.h_v);
    if (W.hdr[0] < 0) return;
    const int slot = slot_ids[j];
    if (slot < 0) return;
    if (slot >= P.n_slots) {
        if (tid == 0 && rb == 0 && h == 0) atomicOr(P.err, kErrSlotRange);
        return;
    }
    const int64_t s0 = cu[j];
    const int len = cu[j + 1] - (int)s0;
    if (len <= 0) return;
    const int G = P.h_v / P.h_k, g = h / G;
    const int K = P.conv_k, C = P.c_conv;
    const int ci0 = W.seq_coff[j], n_ch = W.seq_coff[j + 1] - ci0;
    const int row0 = rb * kRows;
    T* win = reinterpret_cast<T*>(P.window) + ((int64_t)slot * P.n_layers + layer) * (int64_t)(K - 1) * C;
    const int gc0 = 2 * P.h_k * D + h * D + row0;   // first v channel of the block
    const T* vsrc = v + (int64_t)h * D + row0;      // token 0, channel row0
    const int64_t vstride = (int64_t)P.h_v * D;
    float* tile_base = P.state + (((int64_t)slot * P.n_layers + layer) * P.h_v + h) * (int64_t)D * D;

    // ---- load the state block (waves owning a d_k slice).
    f32x4 st[2];
    if (wave < NKS) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const float4 x = *reinterpret_cast<const float4*>(
                tile_base + (int64_t)(row0 + m16) * D + (2 * wave + u) * 16 + q4 * 4);
            st[u] = f32x4{x.x, x.y, x.z, x.w};
        }
    }
    // ---- old v window of the block, then the new window (last conv_k-1 raw
    // inputs of the sequence); this workgroup is the only owner of these
    // channels.
    if (tid < (K - 1) * kRows) {
        const int r = tid / kRows, c = tid % kRows;
        s_win[r][c] = Io<T>::load(win, (int64_t)r * C + gc0 + c);
    }
    __syncthreads();
    if (tid < (K - 1) * kRows) {
        const int r = tid / kRows, c = tid % kRows;
        const int64_t p = s0 + len - (K - 1) + r;
        const float x = p >= s0 ? Io<T>::load(vsrc, p * vstride + c) : s_win[K - 1 + (int)(p - s0)][c];
        Io<T>::store(win, (int64_t)r * C + gc0 + c, x);
    }
    const float* wv = conv_w;   // taps of channel gc0 + c at wv[(gc0 + c) * K + m]

    for (int cc = 0; cc < n_ch; ++cc) {
        const int ci = ci0 + cc;
        const int64_t t0 = s0 + (int64_t)cc * chunk;
        const int L = min(chunk, len - cc * chunk);
        const float* gq = W.qh + ((int64_t)ci * P.h_k + g) * CP * D;
        const float* gk = W.kh + ((int64_t)ci * P.h_k + g) * CP * D;
        const float* gt = W.tq + ((int64_t)ci * P.h_v + h) * CP * CP;
        const float* gp = W.pm + ((int64_t)ci * P.h_v + h) * CP * CP;
        if (tid < CP) s_g[tid] = W.gl[((int64_t)ci * P.h_v + h) * CP + tid];

        // (a) v conv + SiLU for the block's 16 channels.
        for (int e = tid; e < CP * kRows; e += kThreads) {
            const int t = e / kRows, c = e % kRows;
            float y = 0.f;
            if (t < L) {
                float z = 0.f;
                for (int m = 0; m < K; ++m) {
                    const int64_t p = t0 + t - (K - 1) + m;
                    const float x = p >= s0 ? Io<T>::load(vsrc, p * vstride + c)
                                            : s_win[K - 1 + (int)(p - s0)][c];
                    z = fmaf(wv[(int64_t)(gc0 + c) * K + m], x, z);
                }
                y = silu(z);
            }
            s_v[t][c] = y;
        }

        // (b) partial [Q;K] S^T over this wave's d_k slice.
        if (wave < NKS) {
            float sv[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sv[i] = st[0][i];
                sv[4 + i] = st[1][i];
            }
            const Split8 bs = split8(sv);
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) {
                const float* src = (mt < NT ? gq : gk) + (int64_t)((mt % NT) * 16 + m16) * D + wave * 32 + q4 * 4;
                float x[8];
                const float4 x0 = *reinterpret_cast<const float4*>(src);
                const float4 x1 = *reinterpret_cast<const float4*>(src + 16);
                x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
                x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
                const f32x4 acc = mma3(f32x4{0.f, 0.f, 0.f, 0.f}, split8(x), bs);
#pragma unroll
                for (int i = 0; i < 4; ++i) s_xp[wave][mt][(q4 * 4 + i) * 16 + m16] = acc[i];
            }
        }
        __syncthreads();

        // (c) reduce the slices: R = V - gamma * (K S0^T), XQ = gamma * (Q S0^T).
        for (int e = tid; e < CP * kRows; e += kThreads) {
            const int t = e / kRows, r = e % kRows;
            const int tl = t % 16, tt = t / 16;
            float xq = 0.f, xk = 0.f;
#pragma unroll
            for (int w = 0; w < NKS; ++w) {
                xq += s_xp[w][tt][tl * 16 + r];
                xk += s_xp[w][NT + tt][tl * 16 + r];
            }
            const float gam = __expf(s_g[t]);
            s_xq[t][r] = gam * xq;
            s_rt[r][t] = s_v[t][r] - gam * xk;
        }
        __syncthreads();

        // (d) U = T' R, token tile per wave; store U^T and the decayed U^T.
        if (wave < NT) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < CP / 32; ++ks) {
                if (ks * 32 <= wave * 16 + 15) {
                    float x[8];
                    ld8(x, gt + (int64_t)(wave * 16 + m16) * CP + ks * 32 + q4 * 8);
                    const Split8 at = split8(x);
                    ld8(x, &s_rt[m16][ks * 32 + q4 * 8]);
                    acc = mma3(acc, at, split8(x));
                }
            }
            const float glast = s_g[CP - 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = wave * 16 + q4 * 4 + i;
                s_ut[m16][t] = acc[i];
                s_uu[m16][t] = acc[i] * __expf(glast - s_g[t]);
            }
        }
        __syncthreads();

        // (e) O = XQ + P U for the wave's token tile; state update for the
        // wave's d_k tiles: S^T <- exp(g_last) S^T + K^T (decayed U).
        if (wave < NT) {
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = s_xq[wave * 16 + q4 * 4 + i][m16];
#pragma unroll
            for (int ks = 0; ks < CP / 32; ++ks) {
                if (ks * 32 <= wave * 16 + 15) {
                    float x[8];
                    ld8(x, gp + (int64_t)(wave * 16 + m16) * CP + ks * 32 + q4 * 8);
                    const Split8 ap = split8(x);
                    ld8(x, &s_ut[m16][ks * 32 + q4 * 8]);
                    acc = mma3(acc, ap, split8(x));
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = wave * 16 + q4 * 4 + i;
                if (t < L) Io<T>::store(out, ((t0 + t) * P.h_v + h) * D + row0 + m16, acc[i]);
            }
        }
        if (wave < NKS) {
            const float dlast = __expf(s_g[CP - 1]);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int dk0 = (2 * wave + u) * 16;
                f32x4 acc = st[u] * dlast;
#pragma unroll
                for (int ks = 0; ks < CP / 32; ++ks) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = gk[(int64_t)(ks * 32 + q4 * 8 + e) * D + dk0 + m16];
                    const Split8 ak = split8(x);
                    ld8(x, &s_uu[m16][ks * 32 + q4 * 8]);
                    acc = mma3(acc, ak, split8(x));
                }
                st[u] = acc;
            }
        }
        __syncthreads();
    }

    // ---- store the state block back to the slot.
    if (wave < NKS) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
            *reinterpret_cast<float4*>(tile_base + (int64_t)(row0 + m16) * D + (2 * wave + u) * 16 + q4 * 4) =
                make_float4(st[u][0], st[u][1], st[u][2], st[u][3]);
    }
}

template <int D, int CP>
size_t factor_lds_bytes() {
    const size_t a = (size_t)2 * CP * (D + 4) * sizeof(float);
    const size_t b = (size_t)2 * CP * (CP + 1) * sizeof(float);
    return a > b ? a : b;
}

template <int D, int CP, typename T>
hipError_t launch_all(const gdn_pool* pool, Ws W, int32_t layer, int32_t n_seq,
                      const int32_t* cu, const int32_t* slot_ids, int total, int chunk, int mc,
                      const void* q, const void* k, const void* v, const float* a, const float* b,
                      const float* conv_w, void* out, hipStream_t stream) {
    const PoolView& P = pool->view;
    hipLaunchKernelGGL(prefill_prep_kernel, dim3(1), dim3(kPrepThreads), 0, stream, P, W, cu,
                       n_seq, total, chunk, mc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = factor_lds_bytes<D, CP>();
    // More than 64 KiB of dynamic LDS must be enabled per kernel (gfx950 has
    // 160 KiB per CU).
    static bool lds_set = false;
    if (!lds_set) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_factor_kernel<D, CP, T>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        lds_set = true;
    }
    hipLaunchKernelGGL((prefill_factor_kernel<D, CP, T>), dim3(mc, P.h_k), dim3(kThreads), lds,
                       stream, P, W, layer, cu, slot_ids, chunk, static_cast<const T*>(q),
                       static_cast<const T*>(k), a, b, conv_w);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_scan_kernel<D, CP, T>), dim3((D / kRows) * P.h_v * n_seq),
                       dim3(kThreads), 0, stream, P, W, layer, cu, slot_ids, chunk,
                       static_cast<const T*>(v), conv_w, static_cast<T*>(out));
    return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_d(const gdn_pool* pool, Ws W, int32_t layer, int32_t n_seq, const int32_t* cu,
                    const int32_t* slot_ids, int total, int chunk, int mc, const void* q,
                    const void* k, const void* v, const float* a, const float* b,
                    const float* conv_w, void* out, hipStream_t stream) {
    if (chunk == 64)
        return launch_all<D, 64, T>(pool, W, layer, n_seq, cu, slot_ids, total, chunk, mc, q, k, v,
                                    a, b, conv_w, out, stream);
    return launch_all<D, 32, T>(pool, W, layer, n_seq, cu, slot_ids, total, chunk, mc, q, k, v, a,
                                b, conv_w, out, stream);
}

}  // namespace

size_t prefill_workspace_bytes(const gdn_pool* pool, int32_t n_seq, int64_t total_tokens,
                               int32_t chunk) {
    size_t bytes = 0;
    carve(nullptr, pool->view, n_seq, total_tokens, chunk, &bytes);
    return bytes;
}

hipError_t launch_prefill(const gdn_pool* pool, int32_t layer, int32_t n_seq,
                          const int32_t* cu_seqlens, const int32_t* slot_ids,
                          int64_t total_tokens, int32_t chunk, const void* q, const void* k,
                          const void* v, const float* a, const float* b, const float* conv_w,
                          void* out, void* workspace, hipStream_t stream) {
    const PoolView& P = pool->view;
    size_t bytes = 0;
    Ws W = carve(workspace, P, n_seq, total_tokens, chunk, &bytes);
    const int64_t mc = max_chunks(n_seq, total_tokens, chunk);
    if (mc > INT32_MAX || n_seq > 65535) return hipErrorNotSupported;
    const bool bf = pool->desc.io_dtype == GDN_BF16;
    const int total = (int)total_tokens, m = (int)mc;
    switch (P.d) {
#define GDN_CASE(DD)                                                                             \
    case DD:                                                                                     \
        return bf ? launch_d<DD, uint16_t>(pool, W, layer, n_seq, cu_seqlens, slot_ids, total,   \
                                           chunk, m, q, k, v, a, b, conv_w, out, stream)         \
                  : launch_d<DD, float>(pool, W, layer, n_seq, cu_seqlens, slot_ids, total,      \
                                        chunk, m, q, k, v, a, b, conv_w, out, stream);
        GDN_CASE(32)
        GDN_CASE(64)
        GDN_CASE(128)
#undef GDN_CASE
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace gdn
