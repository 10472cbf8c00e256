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
// Kernels, stream-ordered, no host synchronisation:
//   prep   (1 workgroup)             chunk map and scan order from the device
//                                    cu_seqlens (only with more than 64
//                                    sequences; otherwise the factor kernel
//                                    builds them itself);
//   factor (chunk x q/k head)        conv+SiLU, q/k normalisation, KK^T and QK^T
//                                    on bf16 MFMA, T' and P per value head;
//   scan   (seq x v head x 16 rows)  the serial chunk carry on bf16 MFMA, the
//                                    state block kept in registers; sequences
//                                    taken longest first, each spread over
//                                    all XCDs.
// Every MFMA operand that is not an exact bf16 value is split as hi + lo bf16
// and multiplied as hi*hi + hi*lo + lo*hi (fp32 accumulate), which keeps the
// chunked result within fp32-recurrence accuracy.  The factor kernel writes
// the scan's chunk operands (Q^, K^, T', P) already split and in MFMA fragment
// order, so the scan's serial loop only splits what it produces itself; the
// transposed K^ of the state update is read from LDS with the gfx950
// transposing load instead of being stored twice.
#include <algorithm>
#include <mutex>

#include "gdn_common.h"
#include "mfma_split.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;          // state rows (d_v) per scan workgroup
constexpr float kLogDecayMin = -87.f;

// ------------------------------------------------------------ MFMA helpers

// Scatter four consecutive k values (hi and lo) into lane `dl`, elements
// e0..e0+3, of B fragment f.
__device__ __forceinline__ void store_frag4(bf16x8* base, int f, int dl, int e0, const float* x) {
    bf16x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
        bf16x2 hh, ll;
        split2(x[i], x[i + 1], hh, ll);
        h[i] = hh[0];
        h[i + 1] = hh[1];
        l[i] = ll[0];
        l[i + 1] = ll[1];
    }
    *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(base + f * kFragVecs + dl) + e0) = h;
    *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(base + f * kFragVecs + 64 + dl) + e0) = l;
}

// ----------------------------------------------- 16x16 fp32 blocks in LDS

// acc + X Z for 16x16 fp32 blocks in LDS (row stride LT floats), on one
// wave's matrix cores in fp32 (four 16x16x4 steps): lane (m, q) reads
// X[m][k0+q] and Z[k0+q][m] and holds rows 4q..4q+3 of column m of the
// result.
template <int LT>
__device__ __forceinline__ f32x4 blk_mfma(f32x4 acc, const float* X, const float* Z, int lane) {
    const int m = lane & 15, q = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[m * LT + k0 + q], Z[(k0 + q) * LT + m], acc, 0, 0, 0);
    return acc;
}
// Stores a result of blk_mfma (times s) into a 16x16 block.
template <int LT>
__device__ __forceinline__ void blk_store(float* Y, f32x4 v, float s, int lane) {
    const int m = lane & 15, q = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) Y[(4 * q + i) * LT + m] = s * v[i];
}

// Orders one wave's LDS writes before its later LDS reads of other lanes'
// values (a wave's LDS operations complete in order; the fences keep the
// compiler from moving accesses across).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// --------------------------------------------------------------- workspace

// Fragment counts per (chunk, head): CP tokens per chunk (padded), NT = CP/16
// token tiles, NKS = D/32 k-steps over d_k, NKC = CP/32 k-steps over tokens.
struct Geom {
    int D, CP, NT, NKS, NKC;
    int nqk() const { return 2 * NT * NKS; }       // Q^ and K^ rows (A of [Q;K] S0^T)
    int ntp() const { return 2 * NT * NKC; }       // T' and P
};

struct Ws {
    int32_t* hdr;        // [0]: number of chunks, or -1 if cu_seqlens is malformed
    int32_t* seq_coff;   // [n_seq+1] first global chunk of each sequence
    int4* crec;          // [max_chunks][2] per chunk: {sequence, slot, s0, len}, {position, 0, 0, 0}
    int4* srec;          // [n_seq][2] sequences in scan order: {sequence, slot, s0, len}, {first chunk, chunks, 0, 0}
    bf16x8* qkf;         // [max_chunks][h_k][nqk fragments]
    bf16x8* tpf;         // [max_chunks][h_v][ntp fragments]; all-zero ones unwritten
    float* gl;           // [max_chunks][h_v][2][CP] per token: gamma = exp(g), then
                         // eta = exp(g_last - g) (g: cumulative log-decay in the chunk)
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int64_t max_chunks(int32_t n_seq, int64_t total, int32_t chunk) {
    return (total + chunk - 1) / chunk + n_seq;
}

int padded_chunk(int32_t chunk) { return chunk < 32 ? 32 : chunk; }

Geom geom(int D, int chunk) {
    const int CP = padded_chunk(chunk);
    return Geom{D, CP, CP / 16, D / 32, CP / 32};
}

Ws carve(void* base, const PoolView& P, int32_t n_seq, int64_t total, int32_t chunk,
         size_t* bytes) {
    const int64_t mc = max_chunks(n_seq, total, chunk);
    const Geom gm = geom(P.d, chunk);
    const size_t fb = (size_t)kFragVecs * 16;  // bytes per fragment
    size_t off = 0;
    auto take = [&](size_t n) {
        const size_t o = off;
        off += align256(n);
        return o;
    };
    const size_t o_hdr = take(256);
    const size_t o_coff = take((size_t)(n_seq + 1) * 4);
    const size_t o_cseq = take((size_t)mc * 2 * sizeof(int4));
    const size_t o_srec = take((size_t)n_seq * 2 * sizeof(int4));
    const size_t o_qk = take((size_t)mc * P.h_k * gm.nqk() * fb);
    const size_t o_tp = take((size_t)mc * P.h_v * gm.ntp() * fb);
    const size_t o_g = take((size_t)mc * P.h_v * 2 * gm.CP * 4);
    *bytes = off;
    char* b = static_cast<char*>(base);
    Ws w;
    w.hdr = reinterpret_cast<int32_t*>(b + o_hdr);
    w.seq_coff = reinterpret_cast<int32_t*>(b + o_coff);
    w.crec = reinterpret_cast<int4*>(b + o_cseq);
    w.srec = reinterpret_cast<int4*>(b + o_srec);
    w.qkf = reinterpret_cast<bf16x8*>(b + o_qk);
    w.tpf = reinterpret_cast<bf16x8*>(b + o_tp);
    w.gl = reinterpret_cast<float*>(b + o_g);
    return w;
}

// ------------------------------------------------------------------- prep

// One workgroup: check cu_seqlens, count chunks per sequence, prefix-sum them
// and write each chunk's record (its sequence, slot, start, length and
// position), so a factor workgroup finds all of it with one load.  A malformed cu_seqlens marks
// the workspace invalid (the other kernels then do nothing) and sets the
// sticky error bit.  It also writes one record per sequence in the order the
// scan takes them: most chunks first (ties by index) when there are at most
// kSortMax sequences, else in index order.  The scan's serial chain is
// as long as its sequence, so starting the longest chains first keeps short
// ones from leaving a long one alone at the end.
constexpr int kPrepThreads = 1024;
constexpr int kSortMax = 1024;
constexpr int kFusedPrepMax = 64;   // up to this many sequences the factor kernel does the prep

__global__ __launch_bounds__(kPrepThreads) void prefill_prep_kernel(
    PoolView P, Ws W, const int32_t* __restrict__ cu, const int32_t* __restrict__ slot_ids, int n_seq,
    int total, int chunk, int max_chunks) {
    constexpr int kCoffLds = 4096;   // chunk offsets kept in LDS up to this many sequences
    __shared__ int part[kPrepThreads];
    __shared__ int s_coff[kCoffLds + 1];
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
    const bool in_lds = n_seq <= kCoffLds;
    for (int j = j0; j < j1; ++j) {
        W.seq_coff[j] = c;
        if (in_lds) s_coff[j] = c;
        c += (cu[j + 1] - cu[j] + chunk - 1) / chunk;
    }
    if (tid == 0) {
        W.seq_coff[n_seq] = n_chunks;
        if (in_lds) s_coff[n_seq] = n_chunks;
        W.hdr[0] = n_chunks;
    }
    __syncthreads();
    // Sequence records in scan order: rank = number of sequences that come
    // before j (more chunks, or as many and a lower index).
    for (int j = tid; j < n_seq; j += kPrepThreads) {
        const int c0 = in_lds ? s_coff[j] : W.seq_coff[j];
        const int nj = (in_lds ? s_coff[j + 1] : W.seq_coff[j + 1]) - c0;
        int rank = j;
        if (n_seq <= kSortMax) {   // implies in_lds
            rank = 0;
            for (int i = 0; i < n_seq; ++i) {
                const int ni = s_coff[i + 1] - s_coff[i];
                rank += (ni > nj) | ((ni == nj) & (i < j));
            }
        }
        const int s = cu[j];
        W.srec[2 * rank] = make_int4(j, slot_ids[j], s, cu[j + 1] - s);
        W.srec[2 * rank + 1] = make_int4(c0, nj, 0, 0);
    }
    // Chunk records, one thread per chunk: the owning sequence is the j with
    // coff[j] <= chunk < coff[j+1] (binary search; empty sequences own none).
    for (int ch = tid; ch < n_chunks; ch += kPrepThreads) {
        int lo = 0, hi = n_seq;   // coff[lo] <= ch < coff[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            const int v = in_lds ? s_coff[mid] : W.seq_coff[mid];
            if (v <= ch) lo = mid;
            else hi = mid;
        }
        const int s = cu[lo];
        W.crec[2 * ch] = make_int4(lo, slot_ids[lo], s, cu[lo + 1] - s);
        W.crec[2 * ch + 1] = make_int4(ch - (in_lds ? s_coff[lo] : W.seq_coff[lo]), 0, 0, 0);
    }
}

// ------------------------------------------------------------- raw loads

// 16 bytes of raw activations (8 bf16 or 4 fp32) converted to fp32.
template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
    static constexpr int N = 8;
    __device__ static __forceinline__ float at(const uint4& u, int i) {
        const uint32_t w = (i >> 1) == 0 ? u.x : (i >> 1) == 1 ? u.y : (i >> 1) == 2 ? u.z : u.w;
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ static __forceinline__ void load(float* dst, const uint16_t* src) {
        const uint4 u = *reinterpret_cast<const uint4*>(src);
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = at(u, i);
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    __device__ static __forceinline__ float at(const uint4& u, int i) {
        return __uint_as_float(i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w);
    }
    __device__ static __forceinline__ void load(float* dst, const float* src) {
        const uint4 u = *reinterpret_cast<const uint4*>(src);
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = at(u, i);
    }
};

// ------------------------------------------------------------------ factor

// grid (max_chunks, h_k), 256 threads; with fused_n_seq > 0 (at most 64
// sequences) each workgroup finds its chunk from cu_seqlens itself, else it
// reads the prep kernel's chunk record.  The q|k channels of the group are
// staged in NPASS passes (1: all 2D at once, the shortest chain for grids of
// one round; 2: q, then k, in half the LDS, so that three workgroups fit on
// a CU).  KC > 0: conv taps fixed at compile time (must equal conv_k); 0:
// runtime.  NW = 8 waves (one pass, grids of at most one workgroup per CU):
// two groups of four waves solve two value heads side by side, and the
// fragment phase splits q (waves 0-3) from k (waves 4-7).
template <int D, int CP, int KC, int NPASS, int NW, typename T>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : (NPASS == 2 ? 3 : 2)) void prefill_factor_kernel(
    PoolView P, Ws W, int layer, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ slot_ids, int chunk, const T* __restrict__ q,
    const T* __restrict__ k, const float* __restrict__ a, const float* __restrict__ b,
    const float* __restrict__ conv_w, Ckpt ck, int fused_n_seq, int total, int max_chunks) {
    static_assert(NPASS == 1 || NPASS == 2, "staging passes");
    static_assert(NW == 4 || (NW == 8 && NPASS == 1), "waves per workgroup");
    constexpr int NTH = 64 * NW;       // threads
    constexpr int HP = NW / 4;         // value heads solved side by side
    constexpr int CW = 2 * D / NPASS;  // q|k channels staged per pass
    constexpr int LD = CW + 4;         // row of the staged lines (floats)
    constexpr int LT = CP + 4;         // padded row of A, T, P (16-byte aligned)
    constexpr int NT = CP / 16;        // token tiles
    constexpr int NKS = D / 32;        // k-steps over d_k
    constexpr int NKC = CP / 32;       // k-steps over tokens
    constexpr int NQK = 2 * NT * NKS, NTP = 2 * NT * NKC;
    constexpr int VN = Vec<T>::N;
    // Dynamic LDS, reused phase by phase (factor_lds_bytes):
    //   per pass:  raw rows [K-1+CP][LD] of its channels, row r <-> position
    //              t0-(K-1)+r, overwritten in place by the conv+SiLU outputs
    //              (row t) and normalised;
    //   then       the K^ fragments [NT*NKS] (B operands of KK^T, QK^T);
    //   then       per head of the round, A [CP][LT] and T [CP][LT]; P goes
    //              over A once T is done; with two groups, the exchanged
    //              KK^T and QK^T tiles after them.
    extern __shared__ __align__(16) float smem[];
    float* xr = smem;
    constexpr int KM = KC > 0 ? KC : kMaxConvK;   // compile-time tap bound
    constexpr int kMaxGroup = 4;                   // value heads per group kept in LDS
    // Cumulative log-decay in fp64: with a -> 0 (log a down to the clamp)
    // |g| reaches hundreds within a chunk, where fp32 would keep only ~1e-5
    // of the differences g_t - g_s that the decays are made of.
    __shared__ __align__(16) double s_gg[kMaxGroup][CP];
    __shared__ __align__(16) float s_bb[kMaxGroup][CP];
    __shared__ float s_la[kMaxGroup][CP];

    // (the wave index through readfirstlane: known uniform, so conditions on
    // it compile to scalar branches)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m16 = lane & 15, q4 = lane >> 4;
    const int gi = HP == 2 ? wave >> 2 : 0;   // wave group
    const int lw = wave & 3;                  // wave in its group
    const int gt = tid & 255;                 // thread in its group
    const int ci = blockIdx.x, g = blockIdx.y;
    // q|k channel x of the group -> its conv/window channel
    const auto conv_ch = [&](int x) { return x < D ? g * D + x : P.h_k * D + g * D + (x - D); };
    // The conv taps of this thread's channel in every pass, fetched first:
    // they do not depend on the chunk.
    float cw[NPASS][KM];
    {
        const int Kw = KC > 0 ? KC : P.conv_k;
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass)
#pragma unroll
            for (int m = 0; m < KM; ++m)
                cw[pass][m] = m < Kw ? conv_w[(int64_t)conv_ch(pass * CW + tid % CW) * Kw + m] : 0.f;
    }
    int j, slot, len, cpos;   // sequence, its slot and length, chunk index inside it
    int64_t s0;
    if (fused_n_seq > 0) {
        // At most 64 sequences: no prep launch.  Wave 0 of every workgroup
        // checks cu_seqlens and prefix-sums the chunk counts (one lane per
        // sequence) and finds the sequence owning chunk ci; workgroup (0, 0)
        // also writes the header and the scan's sequence records (as the
        // prep kernel does).
        __shared__ int s_rec[6];
        if (wave == 0) {
            const int n = fused_n_seq;
            const bool in = lane < n;
            const int cs = in ? cu[lane] : 0, ce = in ? cu[lane + 1] : 0;
            const int sl = in ? slot_ids[lane] : 0;
            const bool bad_j = in && (cs < 0 || ce < cs || ce > total);
            const int nj = in && !bad_j ? (ce - cs + chunk - 1) / chunk : 0;
            int incl = nj;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {   // inclusive prefix sum over the wave
                const int y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            const int excl = incl - nj, n_chunks = __shfl(incl, 63);
            const bool bad = __any(bad_j) || __shfl(cs, 0) != 0 || __shfl(ce, n - 1) != total ||
                             n_chunks > max_chunks;
            const unsigned long long own = __ballot(in && ci >= excl && ci < incl);
            const int jo = own ? __ffsll((unsigned long long)own) - 1 : 0;
            const int o_cs = __shfl(cs, jo), o_ce = __shfl(ce, jo), o_sl = __shfl(sl, jo);
            const int o_ex = __shfl(excl, jo);
            if (ci == 0 && g == 0) {
                int rank = 0;   // scan order: more chunks first, ties by index
                for (int i = 0; i < n; ++i) {
                    const int ni = __shfl(nj, i);
                    rank += (ni > nj) | ((ni == nj) & (i < lane));
                }
                if (lane == 0) {
                    W.hdr[0] = bad ? -1 : n_chunks;
                    if (bad) atomicOr(P.err, kErrSeqlens);
                }
                if (in && !bad) {
                    W.srec[2 * rank] = make_int4(lane, sl, cs, ce - cs);
                    W.srec[2 * rank + 1] = make_int4(excl, nj, 0, 0);
                }
            }
            if (lane == 0) {
                s_rec[0] = bad || !own;
                s_rec[1] = jo;
                s_rec[2] = o_sl;
                s_rec[3] = o_cs;
                s_rec[4] = o_ce - o_cs;
                s_rec[5] = ci - o_ex;
            }
        }
        __syncthreads();
        if (s_rec[0]) return;
        j = s_rec[1];
        slot = s_rec[2];
        s0 = s_rec[3];
        len = s_rec[4];
        cpos = s_rec[5];
    } else {
        const int4 rec0 = W.crec[2 * ci], rec1 = W.crec[2 * ci + 1];   // read with the count
        const int n_chunks = W.hdr[0];
        if (ci >= n_chunks) return;        // also when the workspace is invalid (-1)
        j = rec0.x;
        slot = rec0.y;
        s0 = rec0.z;
        len = rec0.w;
        cpos = rec1.x;
    }
    if (slot < 0 || slot >= P.n_slots) return;
    const int64_t t0 = s0 + (int64_t)cpos * chunk;
    const int L = min(chunk, len - cpos * chunk); // valid tokens in this chunk
    const int K = KC > 0 ? KC : P.conv_k, C = P.c_conv, G = P.h_v / P.h_k;
    T* win = reinterpret_cast<T*>(P.window) + ((int64_t)slot * P.n_layers + layer) * (int64_t)(K - 1) * C;

    // ---- a and b of the chunk's tokens for every value head of the group,
    // fetched with the staging loads (unconditional, positions clamped into
    // the chunk; log a clamped; zero past L).  G * CP <= NTH.
    static_assert(kMaxGroup * 64 <= NTH, "one a/b value per thread");
    const int ab_hl = min(tid / CP, G - 1), ab_t = tid % CP;
    float ab_a, ab_b;
    {
        const int64_t tok = t0 + min(ab_t, L - 1);
        ab_a = a[tok * P.h_v + g * G + ab_hl];
        ab_b = b[tok * P.h_v + g * G + ab_hl];
    }

    // ---- per pass: stage the raw rows, conv + SiLU in place, normalise, and
    // split the wave's token tile into MFMA fragments.  Channel c of pass p
    // is q|k channel p*CW + c (q below D).  Wave w builds the fragments of
    // token tile w, so the A operands of KK^T and QK^T stay in its
    // registers; the K^ fragments also go to LDS as the B operands of every
    // tile row.
    Frag fq[NKS], fk[NKS];
    // Raw rows with 16-byte loads, every pass's issued here, before the
    // first is used (source pointer selected, position clamped into the
    // chunk), so the staging costs one round trip: window rows before the
    // sequence start, token L-1 again past the chunk's valid tokens.
    const int nrow = K - 1 + CP;
    constexpr int vpr = CW / VN;
    constexpr int NST = ((KM - 1 + CP) * vpr + NTH - 1) / NTH;
    static_assert(NTH % vpr == 0, "a thread keeps its column across iterations");
    constexpr int RPI = NTH / vpr;                    // rows per iteration
    uint4 raw[NPASS][NST];
    {
        const int cv0 = (tid % vpr) * VN, r0 = tid / vpr;
        const int64_t tstride = (int64_t)P.h_k * D;       // elements between tokens
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            const int x0 = pass * CW + cv0;               // q|k channel of the column
            const T* tok_base = (x0 < D ? q + x0 : k + (x0 - D)) + t0 * tstride + g * D;
            const T* win_base = win + conv_ch(x0);
#pragma unroll
            for (int it = 0; it < NST; ++it) {
                const int r = min(r0 + it * RPI, nrow - 1);
                const int dt = min(r - (K - 1), L - 1);       // token offset from t0, clamped into the chunk
                const int64_t p = t0 + dt;
                const T* ps = p >= s0 ? tok_base + (int64_t)dt * tstride
                                      : win_base + (int64_t)(K - 1 + (int)(p - s0)) * C;
                raw[pass][it] = *reinterpret_cast<const uint4*>(ps);
            }
        }
    }
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int xb = pass * CW;   // first q|k channel of the pass
        // a/b arrive with the first staging loads; consume them only now
        if (pass == 0 && tid < G * CP) {
            s_la[ab_hl][ab_t] = ab_t < L ? fmaxf(__logf(ab_a), kLogDecayMin) : 0.f;
            s_bb[ab_hl][ab_t] = ab_t < L ? ab_b : 0.f;
        }
#pragma unroll
        for (int it = 0; it < NST; ++it) {
            const int e = tid + it * NTH;
            if (e < nrow * vpr) {
                // rows past the chunk's valid tokens hold token L-1 (the load
                // was clamped): only the conv outputs of padding tokens read
                // them, and those never reach a valid output or the state
                // (their b is zero, so their rows of A and of T' are zero)
                const int r = e / vpr, cv = (e % vpr) * VN;
                float x[VN];
#pragma unroll
                for (int i = 0; i < VN; ++i) x[i] = Vec<T>::at(raw[pass][it], i);
#pragma unroll
                for (int i = 0; i < VN; i += 4)
                    *reinterpret_cast<float4*>(xr + r * LD + cv + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
            }
        }
        __syncthreads();
        // The sequence's first chunk owns the window of these channels: store
        // the last conv_k-1 raw inputs of the sequence (old window rows come
        // from LDS).
        if (cpos == 0) {
            for (int e = tid; e < (K - 1) * CW; e += NTH) {
                const int m = e / CW, c = e % CW, x = xb + c;
                const int64_t pp = s0 + len - (K - 1) + m;
                const float v = pp >= s0 ? Io<T>::load(x < D ? q : k, (pp * P.h_k + g) * D + (x < D ? x : x - D))
                                         : xr[(int)(K - 1 + (pp - s0)) * LD + c];
                Io<T>::store(win, (int64_t)m * C + conv_ch(x), v);
            }
        }
        // A checkpoint after this chunk (full, ending on a multiple of the
        // checkpoint interval) holds these channels' last conv_k-1 raw rows.
        if (ck.every_chunks > 0 && L == chunk && (cpos + 1) % ck.every_chunks == 0) {
            const int m = (cpos + 1) / ck.every_chunks - 1;
            const int cs = m < ck.off[j + 1] - ck.off[j] ? ck.slots[ck.off[j] + m] : -1;
            if (cs >= 0 && cs < P.n_slots) {
                T* cwin = reinterpret_cast<T*>(P.window) + ((int64_t)cs * P.n_layers + layer) * (int64_t)(K - 1) * C;
                for (int e = tid; e < (K - 1) * CW; e += NTH) {
                    const int r = e / CW, c = e % CW;
                    Io<T>::store(cwin, (int64_t)r * C + conv_ch(xb + c), xr[(chunk + r) * LD + c]);
                }
            }
        }
        // ---- conv + SiLU: one channel and TPH consecutive tokens per thread.
        // y_t lands in row t, which no later token of the channel reads; the
        // K-1 rows past the thread's slice are the next slice's first outputs,
        // so they are read into registers before a barrier.
        {
            constexpr int TPH = CP / (NTH / CW);
            static_assert(NTH % CW == 0 && TPH >= 1, "token slices of the conv");
            const int c = tid % CW, t0c = (tid / CW) * TPH;
            const float* w = cw[pass];
            float line[KM - 1], tail[KM - 1];
#pragma unroll
            for (int m = 0; m < KM - 1; ++m) {
                line[m] = m < K - 1 ? xr[(t0c + m) * LD + c] : 0.f;
                tail[m] = m < K - 1 && TPH < CP ? xr[(t0c + TPH + m) * LD + c] : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < TPH; ++i) {
                // raw row t0c+i+K-1: in LDS (this slice's, or with one slice
                // every row), or one of the saved tail rows
                float x = 0.f;
                if (i + K - 1 < TPH || TPH == CP) {
                    x = xr[(t0c + i + K - 1) * LD + c];
                } else {
#pragma unroll
                    for (int m = 0; m < KM - 1; ++m)
                        if (i + K - 1 - TPH == m) x = tail[m];
                }
                float z = 0.f;
#pragma unroll
                for (int m = 0; m < KM - 1; ++m)
                    if (m < K - 1) z = fmaf(w[m], line[m], z);
                z = fmaf(w[K - 1], x, z);
                xr[(t0c + i) * LD + c] = silu(z);   // padding tokens too (see the staging)
#pragma unroll
                for (int m = 0; m < KM - 1; ++m)
                    line[m] = (m == K - 2) ? x : (m < K - 2 ? line[m + 1] : line[m]);
            }
        }
        __syncthreads();
        // ---- normalisation and fragments (qk, tile = wave, ks), lane (m, q):
        // token tile*16+m, d_k {32ks+4q+i, 32ks+16+4q+i} (the d_k order in
        // which the scan holds its state).  The four lanes of a token
        // (q = 0..3, 16 lanes apart) hold all of its D channels of q (h = 0)
        // or k (h = 1): they add up their sums of squares, scale, and split
        // each value once.  The scan builds the state update's K^T operand
        // from these itself (LDS transpose reads).  The workspace is written
        // with non-temporal stores: only the scan, a later launch, reads it,
        // and lines left dirty in L2 would lengthen the write-back at the end
        // of this launch.
        if (lw < NT) {
            bf16x8* gqk = W.qkf + ((int64_t)ci * P.h_k + g) * NQK * kFragVecs;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h * D < xb || h * D >= xb + CW) continue;   // not in this pass
                if (HP == 2 && h != gi) continue;               // group 0: q, group 1: k
                float x[NKS][8];
                float sq = 0.f;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const float* row = xr + (lw * 16 + m16) * LD + (h * D - xb) + ks * 32 + q4 * 4;
                    ld4x2(x[ks], row, row + 16);
                }
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) sq = fmaf(x[ks][e], x[ks][e], sq);
                sq += __shfl_xor(sq, 16);
                sq += __shfl_xor(sq, 32);
                const float rs = (h ? 1.0f : P.q_scale) / sqrtf(sq + P.eps);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[ks][e] *= rs;
                    const Frag f = split8(x[ks]);
                    store_frag_nt(gqk, (h * NT + lw) * NKS + ks, lane, f);
                    if (h) fk[ks] = f;
                    else fq[ks] = f;
                }
            }
        }
        __syncthreads();   // the next pass (or the fragments below) overwrite the rows
    }
    bf16x8* const lfr = reinterpret_cast<bf16x8*>(smem);   // [NT*NKS] K^ fragments
    if (lw < NT && (HP == 1 || gi == 1)) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) store_frag(lfr, lw * NKS + ks, lane, fk[ks]);
    }
    __syncthreads();
    // Per head of a round: A and T (P over A) of group gi's head.
    const auto sA_of = [&](int gg) { return smem + gg * 2 * CP * LT; };
    f32x4* const xch = reinterpret_cast<f32x4*>(smem + HP * 2 * CP * LT);   // [2][NT][NT][64]

    // ---- KK^T and QK^T lower-triangular tiles: wave w takes tile row w.  A
    // and B are the same split fragments (one d_k order on both sides).  With
    // two groups, group 1 (which holds K^) computes KK^T and group 0 (Q^)
    // QK^T; each passes its tiles to the other through LDS.
    f32x4 kk[NT], qk[NT];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
        kk[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        qk[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int ti = lw;  // tile row
    // Cumulative log-decay of value head hl of the group by wave hl (the
    // first waves have the fewest tile rows below).
    if (wave < G) {
        double la = lane < CP ? (double)s_la[wave][lane] : 0.0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {   // inclusive prefix sum (CP <= 64)
            const double y = __shfl_up(la, o);
            if (lane >= o) la += y;
        }
        if (lane < CP) s_gg[wave][lane] = la;
    }
    if (ti < NT) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int jt = 0; jt < NT; ++jt) {
                if (jt <= ti) {
                    const Frag bk = load_frag(lfr, jt * NKS + ks, lane);
                    if (HP == 1) {
                        kk[jt] = mma3(kk[jt], fk[ks], bk);
                        qk[jt] = mma3(qk[jt], fq[ks], bk);
                    } else if (gi == 1) {
                        kk[jt] = mma3(kk[jt], fk[ks], bk);
                    } else {
                        qk[jt] = mma3(qk[jt], fq[ks], bk);
                    }
                }
            }
        }
        if (HP == 2) {
#pragma unroll
            for (int jt = 0; jt < NT; ++jt)
                if (jt <= ti) xch[((gi * NT + ti) * NT + jt) * 64 + lane] = gi ? kk[jt] : qk[jt];
        }
    }
    __syncthreads();   // the fragment region is reused below
    if (HP == 2 && ti < NT) {
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
            if (jt <= ti) {
                const f32x4 x = xch[(((1 - gi) * NT + ti) * NT + jt) * 64 + lane];
                if (gi) qk[jt] = x;
                else kk[jt] = x;
            }
        }
    }

    // ---- per value head of the group (HP at a time, group gi takes head
    // hl0 + gi): decay, A, T = (I+A)^-1, T', P.  Every wave runs every
    // barrier; a group without a head in the last round (odd G) idles.
    for (int hl0 = 0; hl0 < G; hl0 += HP) {
        const int hl = min(hl0 + gi, G - 1);
        const bool act = hl0 + gi < G;   // uniform per wave
        const int hv = g * G + hl;
        const double* s_g = s_gg[hl];   // cumulative log-decay (zero past L)
        const float* s_b = s_bb[hl];    // b (zero past L)
        float* const sA = sA_of(gi);
        float* const sT = sA + CP * LT;
        float* const sP = sA;
        // A (strictly lower) into LDS, P (lower incl. diagonal) into
        // registers until T is done.  The lane's four rows share their g and b
        // (one vector read each); blocks above the diagonal are plain zeros.
        float pvr[NT][4];
        // The column index goes through an empty asm: the s < t and s <= t
        // lane masks below are then recomputed per head (one compare each)
        // instead of being hoisted out of the loop and spilled (two lane
        // reads each).
        int m16h = m16;
        asm volatile("" : "+v"(m16h));
        if (act && ti < NT) {
            const double2 ga = *reinterpret_cast<const double2*>(s_g + ti * 16 + q4 * 4);
            const double2 gb = *reinterpret_cast<const double2*>(s_g + ti * 16 + q4 * 4 + 2);
            const float4 bt4 = *reinterpret_cast<const float4*>(s_b + ti * 16 + q4 * 4);
            const double gt[4] = {ga.x, ga.y, gb.x, gb.y};
            const float bt[4] = {bt4.x, bt4.y, bt4.z, bt4.w};
#pragma unroll
            for (int jt = 0; jt < NT; ++jt) {
                const int s = jt * 16 + m16h;         // column
                const double gs = s_g[s];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = ti * 16 + q4 * 4 + r;   // row (later token)
                    float av = 0.f, pv = 0.f;
                    if (jt <= ti) {
                        const float dec = __expf(fminf((float)(gt[r] - gs), 0.f));
                        av = s < t ? bt[r] * dec * kk[jt][r] : 0.f;
                        pv = s <= t ? qk[jt][r] * dec : 0.f;
                    }
                    sA[t * LT + s] = av;
                    pvr[jt][r] = pv;
                }
            }
        }
        // T's upper blocks (2b, 2b+1) share a 32-wide k-step with a diagonal
        // block in the T' fragments: zero them, so the fragments need no mask.
        for (int e = gt; act && e < (NT / 2) * 256; e += 256) {
            const int pb = e / 256, r = (e % 256) / 16, c = e % 16;
            sT[(2 * pb * 16 + r) * LT + (2 * pb + 1) * 16 + c] = 0.f;
        }
        __syncthreads();

        // (I+A)^-1, blocked by 16.  Diagonal blocks by forward substitution,
        // one wave per block: lane = 4 * column c + part p; part p owns columns
        // 4p..4p+3 of the block's A rows (read row by row) and the matching
        // rows of T's column c (in registers).  Entries of T not yet computed are still zero, so
        // row r of T is -sum over the whole row of A times T, no predicates.
        if (act && lw < NT) {
            const int blk = lw * 16;
            int c = lane >> 2;   // opaque, like m16h above: its masks stay in the loop
            asm volatile("" : "+v"(c));
            const int pp = lane & 3;
            float tq[4] = {0.f, 0.f, 0.f, 0.f};   // T[blk + 4pp + i][blk + c]
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                // row r of the block's A (this part's four columns), read at
                // its step rather than all up front: 4 registers, not 64
                const float4 a4 = *reinterpret_cast<const float4*>(sA + (blk + r) * LT + blk + 4 * pp);
                const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = fmaf(ar[i], tq[i], acc);
                acc = group_sum<4>(acc);
                const float trc = (r == c) ? 1.f : (r > c ? -acc : 0.f);
#pragma unroll
                for (int i = 0; i < 4; ++i) tq[i] = (4 * pp + i == r) ? trc : tq[i];
                if (pp == 0) sT[(blk + r) * LT + blk + c] = trc;
            }
        }
        __syncthreads();
        // Off-diagonal blocks by block doubling: for each pair of adjacent
        // runs of s blocks (s = 1, then 2 for four blocks), the lower-left
        // part of T is -T_BB L_BA T_AA (L = I + A; runs A above B).  One wave
        // per output block, its 16x16 products on the matrix cores in fp32;
        // the products X = L_BA T_AA that it needs go through A's upper
        // blocks (zero, unused), each private to one wave, within the wave
        // (no workgroup barrier between the two products).
        {
            const auto blkA = [&](int bi, int bj) { return sA + bi * 16 * LT + bj * 16; };
            const auto blkT = [&](int bi, int bj) { return sT + bi * 16 * LT + bj * 16; };
            const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
            const int wu = __builtin_amdgcn_readfirstlane(lw);   // wave in its group, known uniform
            if (act && wu < NT / 2) {   // s = 1: block (2w+1, 2w)
                const int bi = 2 * wu + 1, bj = 2 * wu;
                float* xs = blkA(0, 1 + wu);
                blk_store<LT>(xs, blk_mfma<LT>(zero, blkA(bi, bj), blkT(bj, bj), lane), 1.f, lane);
                wave_lds_sync();
                blk_store<LT>(blkT(bi, bj), blk_mfma<LT>(zero, blkT(bi, bi), xs, lane), -1.f, lane);
            }
            __syncthreads();
            if (act && NT == 4) {
                // s = 2: block (bi, bj) = (2 + w/2, w%2) of T is
                // -(T_{bi,2} X_{2,bj} + T_{bi,3} X_{3,bj}) with
                // X_{m,bj} = A_{m,0} T_{0,bj} + A_{m,1} T_{1,bj}.  T_{0,1} and
                // T_{2,3} are zero, so every wave runs the same products.  The
                // wave's two X blocks go to unused upper blocks: of A,
                // (0,1) (0,2) | (0,3) (1,2) | (1,3) (2,3) for waves 0-2, and of
                // T, (0,2) (0,3) for wave 3.
                const int bi = 2 + wu / 2, bj = wu % 2;
                float* const xb = wu == 3 ? sT : sA;
                float* xs2 = xb + (wu == 2 ? 16 * LT : 0) + (wu == 0 ? 1 : wu == 3 ? 2 : 3) * 16;
                float* xs3 = xb + wu % 3 * 16 * LT + (wu == 2 || wu == 3 ? 3 : 2) * 16;
                f32x4 x2 = blk_mfma<LT>(zero, blkA(2, 0), blkT(0, bj), lane);
                f32x4 x3 = blk_mfma<LT>(zero, blkA(3, 0), blkT(0, bj), lane);
                x2 = blk_mfma<LT>(x2, blkA(2, 1), blkT(1, bj), lane);
                x3 = blk_mfma<LT>(x3, blkA(3, 1), blkT(1, bj), lane);
                blk_store<LT>(xs2, x2, 1.f, lane);
                blk_store<LT>(xs3, x3, 1.f, lane);
                wave_lds_sync();
                f32x4 t = blk_mfma<LT>(zero, blkT(bi, 2), xs2, lane);
                t = blk_mfma<LT>(t, blkT(bi, 3), xs3, lane);
                blk_store<LT>(blkT(bi, bj), t, -1.f, lane);
            }
            __syncthreads();
        }
        // P over A (A and the block products kept in its upper part are done).
        if (act && ti < NT) {
#pragma unroll
            for (int jt = 0; jt < NT; ++jt)
#pragma unroll
                for (int r = 0; r < 4; ++r) sP[(ti * 16 + q4 * 4 + r) * LT + jt * 16 + m16] = pvr[jt][r];
        }
        __syncthreads();
        // T' = T diag(b) and P fragments: (tp, tile, kc), lane (m, q): row
        // tile*16+m, cols 32kc+8q+e.  Both are lower triangular: fragments with
        // kc > tile/2 are all zero and are not written (the scan never fetches
        // them); inside the others T's upper part is zero (see above).
        bf16x8* gtp = W.tpf + ((int64_t)ci * P.h_v + hv) * NTP * kFragVecs;
        for (int f = lw; act && f < NTP; f += 4) {
            const int tp = f / (NT * NKC), tile = (f / NKC) % NT, kc = f % NKC;
            if (kc > tile / 2) continue;
            float x[8];
            ld8(x, (tp ? sP : sT) + (tile * 16 + m16) * LT + kc * 32 + q4 * 8);
            if (tp == 0) {   // T' = T diag(b); T is zero above the diagonal here
                float bb[8];
                ld8(bb, s_b + kc * 32 + q4 * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] *= bb[e];
            }
            store_frag_nt(gtp, f, lane, split8(x));
        }
        if (act && gt < 2 * CP) {   // gamma_t, then eta_t = exp(g_last - g_t), from fp64 g
            const int t = gt % CP;
            const float e = gt < CP ? (float)s_g[t] : (float)(s_g[CP - 1] - s_g[t]);
            __builtin_nontemporal_store(__expf(e), W.gl + ((int64_t)ci * P.h_v + hv) * 2 * CP + gt);
        }
        __syncthreads();
    }
}

// -------------------------------------------------------------------- scan

// One workgroup per (sequence, value head, block of 16 state rows), 256
// threads, serial over the sequence's chunks.  Per chunk (three phases):
//   1. wave w < CP/16 takes token tile w: X_K = K S0^T and X_Q = Q S0^T for
//      its 16 tokens (B operand: the state block, published split in LDS,
//      read once for both); R = V - diag(gamma) X_K goes to LDS as B
//      fragments and XQ = diag(gamma) X_Q stays in registers;
//   2. U = T' R for the tile, published as B fragments with its decayed copy
//      diag(exp(g_last - g)) U;
//   3. O = XQ + P U for the tile is written out; wave w < D/32 updates state
//      tiles 2w, 2w+1 of S^T (d_k x rows), S^T <- exp(g_last) S^T + K^T (decayed
//      U), and republishes them.  K^T comes from the chunk's K^ rows, staged
//      in LDS by phase 1 and read back with transposing loads.
// The next chunk's fragments (registers) are fetched while the current chunk
// computes; raw v rows and g run one chunk further ahead (registers, then a
// second LDS buffer).
template <int D, int CP>
struct ScanLds {
    static constexpr int NKS = D / 32, NKC = CP / 32;
    static constexpr int NRAW = kMaxConvK - 1 + CP;
    // 16-byte vectors
    static constexpr int stf = 0;                              // [NKS] state fragments
    static constexpr int rf = stf + NKS * kFragVecs;           // [NKC] R fragments
    static constexpr int uf = rf + NKC * kFragVecs;            // [NKC] U fragments
    static constexpr int uuf = uf + NKC * kFragVecs;           // [NKC] decayed U fragments
    static constexpr int vec_end = uuf + NKC * kFragVecs;
    // floats, after the fragments
    static constexpr int vv = vec_end * 4;                     // [2][CP][16] conv+SiLU of v
    static constexpr int raw = vv + 2 * CP * kRows;            // [2][NRAW][16] raw v rows
    static constexpr int gg = raw + 2 * NRAW * kRows;          // [2][2][CP] gamma, eta per token
    static constexpr int win = gg + 4 * CP;                    // [kMaxConvK-1][16] old window
    // K^ of the chunk, bf16 planes hi and lo, [CP][D] with the 16-element
    // column groups of each row XOR-swizzled (kswz), so the rows read
    // together by a transpose read fall in disjoint banks.
    static constexpr int KRS = D;
    static constexpr int kn = (win + (kMaxConvK - 1) * kRows + 3) / 4 * 4;
    static constexpr int total = kn + CP * KRS;                // 2 planes of bf16 = CP*KRS floats
    static constexpr size_t bytes = (size_t)total * sizeof(float);
};

// Transposing LDS read (gfx950): lane 16g+j receives element j%4 of the four
// bf16 at the address of lane 16g+4e+j/4, for e = 0..3.
// XOR swizzle (in elements, a multiple of 4) of row `row` of the staged K^
// planes: both the transposing reads and the 8-byte staging writes run at the
// LDS's full rate with it (measured on gfx950 with 8 waves per CU: about 4
// cycles per wave instruction, against 10 for the writes with a 16-element
// swizzle and 13-40 unswizzled).
template <int D>
__device__ __forceinline__ int kswz(int row) {
    return (4 * ((row & 1) | (((row >> 3) & 1) << 1)) + 16 * ((row >> 1) & 7)) & (D - 4);
}
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(bf16x4, r);
}

template <int D, int CP, int KC, typename T>
__global__ __launch_bounds__(kThreads, 2) void prefill_scan_kernel(
    PoolView P, Ws W, int layer, int chunk, const T* __restrict__ v,
    const float* __restrict__ conv_w, T* __restrict__ out, Ckpt ck) {
    using S = ScanLds<D, CP>;
    constexpr int NKS = D / 32;       // 32-wide k-steps over d_k
    constexpr int NT = CP / 16;       // token tiles
    constexpr int NKC = CP / 32;      // 32-wide k-steps over tokens
    constexpr int NQK = 2 * NT * NKS, NTP = 2 * NT * NKC;
    constexpr int NRAW = S::NRAW;
    constexpr int KRS = S::KRS;
    extern __shared__ __align__(16) float smem[];
    bf16x8* s_stf = reinterpret_cast<bf16x8*>(smem) + S::stf;
    bf16x8* s_rf = reinterpret_cast<bf16x8*>(smem) + S::rf;
    bf16x8* s_uf = reinterpret_cast<bf16x8*>(smem) + S::uf;
    bf16x8* s_uuf = reinterpret_cast<bf16x8*>(smem) + S::uuf;
    float* s_v = smem + S::vv;
    float* s_raw = smem + S::raw;
    float* s_g = smem + S::gg;
    float* s_win = smem + S::win;
    __bf16* s_kh = reinterpret_cast<__bf16*>(smem + S::kn);   // K^ hi plane
    __bf16* s_kl = s_kh + CP * KRS;                            // K^ lo plane

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m16 = lane & 15, q4 = lane >> 4;
    // Work units: sequence jj of the scan order, q/k head g, and the G * D/16
    // (value head, row block) pairs of that group.  Consecutive workgroup ids
    // go to different XCDs (round robin over 8).  When the (jj, g) count is a
    // multiple of 8, (jj, g) goes to XCD (jj * h_k + g) % 8 with all of its
    // workgroups, so the row blocks and value heads that read the same chunk
    // operands share that XCD's L2, every sequence is spread over all XCDs,
    // and each XCD starts its units in scan order (longest sequence first).
    constexpr int NRB = D / kRows;
    const int G = P.h_v / P.h_k;
    const int bid = blockIdx.x;
    int jj, g, r;
    if ((gridDim.x / (G * NRB)) % 8 == 0) {
        const int i = bid / 8, ku = (i / (G * NRB)) * 8 + bid % 8;
        jj = ku / P.h_k;
        g = ku % P.h_k;
        r = i % (G * NRB);
    } else {
        jj = bid / (NRB * P.h_v);
        g = (bid / (G * NRB)) % P.h_k;
        r = bid % (G * NRB);
    }
    const int h = g * G + r / NRB, rb = r % NRB;
    if (W.hdr[0] < 0) return;
    const int4 sr0 = W.srec[2 * jj], sr1 = W.srec[2 * jj + 1];
    const int j = sr0.x, slot = sr0.y;
    if (slot < 0) return;
    if (slot >= P.n_slots) {
        if (tid == 0 && rb == 0 && h == 0) atomicOr(P.err, kErrSlotRange);
        return;
    }
    const int64_t s0 = sr0.z;
    const int len = sr0.w;
    if (len <= 0) return;
    const int K = KC > 0 ? KC : P.conv_k, C = P.c_conv;
    constexpr int KM = KC > 0 ? KC : kMaxConvK;   // compile-time tap bound
    const int ci0 = sr1.x, n_ch = sr1.y;
    const int row0 = rb * kRows;
    T* win = reinterpret_cast<T*>(P.window) + ((int64_t)slot * P.n_layers + layer) * (int64_t)(K - 1) * C;
    const int gc0 = 2 * P.h_k * D + h * D + row0;   // first v channel of the block
    const T* vsrc = v + (int64_t)h * D + row0;      // token 0, channel row0
    const int64_t vstride = (int64_t)P.h_v * D;
    float* tile_base = P.state + (((int64_t)slot * P.n_layers + layer) * P.h_v + h) * (int64_t)D * D;

    // Every global access in the chunk loop is unconditional (chunk indices
    // clamped, waves without a tile of their own redo tile NT-1 / NKS-1 and
    // write identical values), so the compiler can count outstanding loads
    // exactly and each prefetch is waited for only where it is used.
    const int tw = wave < NT ? wave : NT - 1;       // token tile of this wave
    const int sw = wave < NKS ? wave : NKS - 1;     // d_k k-step / state tiles of this wave

    // ---- operand fetchers -------------------------------------------------
    Frag fqk[2][NKS];      // Q and K fragments of token tile tw
    Frag ftt[NKC];         // T' fragments of token tile tw
    Frag fpp[NKC];         // P fragments of token tile tw
    // qk = 0: Q^, 1: K^ (both used in phase 1); each is refetched for
    // the next chunk right after its last use.
    auto load_qk = [&](int ci, int qk) {
        const bf16x8* base = W.qkf + ((int64_t)ci * P.h_k + g) * NQK * kFragVecs;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) fqk[qk][ks] = load_frag(base, (qk * NT + tw) * NKS + ks, lane);
    };
    // T' and P fragments through a buffer descriptor over the (chunk, head)
    // block: the all-zero fragments above the diagonal (kc > tw/2) get an
    // offset past its end, which returns zeros without touching memory.
    constexpr int kFragBytes = kFragVecs * 16;
    auto tp_frag = [&](int ci, int tp, Frag* dst) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<bf16x8*>(W.tpf + ((int64_t)ci * P.h_v + h) * NTP * kFragVecs), 0,
            NTP * kFragBytes, 0x00020000);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            const int off = kc <= tw / 2 ? ((tp * NT + tw) * NKC + kc) * kFragBytes : NTP * kFragBytes;
            dst[kc].hi = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off + lane * 16, 0, 0));
            dst[kc].lo = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 1024 + lane * 16, 0, 0));
        }
    };
    auto load_t = [&](int ci) { tp_frag(ci, 0, ftt); };
    auto load_p = [&](int ci) { tp_frag(ci, 1, fpp); };
    // L2 prefetch of a chunk's Q^/K^ and T'/P blocks: the D/16 workgroups of
    // a head (same XCD) each touch their share of its 128-byte lines with one
    // dword load per line.  Issued after the step's last fragment loads and
    // consumed one step later, so no fragment load waits behind it.
    constexpr int LQ = NQK * kFragBytes / 128, LTP = NTP * kFragBytes / 128;
    constexpr int PSH = (LQ + LTP + NRB - 1) / NRB;             // lines per workgroup
    static_assert(PSH <= kThreads, "one prefetch line per thread");
    uint32_t pf_sink = 0, pf_val = 0;
    auto prefetch = [&](int ci) {
        const int li = min(rb * PSH + min(tid, PSH - 1), LQ + LTP - 1);
        const char* p = li < LQ
            ? reinterpret_cast<const char*>(W.qkf + ((int64_t)ci * P.h_k + g) * NQK * kFragVecs) + li * 128
            : reinterpret_cast<const char*>(W.tpf + ((int64_t)ci * P.h_v + h) * NTP * kFragVecs) + (li - LQ) * 128;
        pf_sink ^= pf_val;
        pf_val = *reinterpret_cast<const uint32_t*>(p);
    };
    // Raw v rows of chunk cc (left context first) and its g, fetched into
    // registers: one 16-byte vector per (row, part) and one g per token.  The
    // address is clamped into the sequence, out-of-chunk rows are zeroed after
    // the load.
    constexpr int VN = Vec<T>::N;
    constexpr int kRawVec = kRows / VN;             // vectors per raw row
    constexpr int kRawIt = (NRAW * kRawVec + kThreads - 1) / kThreads;
    uint4 rv[kRawIt];
    float rg = 0.f;
    auto fetch_raw = [&](int cc) {
        const int64_t t0 = s0 + (int64_t)cc * chunk;
#pragma unroll
        for (int it = 0; it < kRawIt; ++it) {
            const int e = tid + it * kThreads;
            const int r = e / kRawVec, cv = (e % kRawVec) * VN;
            const int64_t p = t0 - (K - 1) + r;
            const int64_t pc = p < s0 ? s0 : (p >= s0 + len ? s0 + len - 1 : p);
            rv[it] = *reinterpret_cast<const uint4*>(vsrc + pc * vstride + cv);
        }
        rg = W.gl[((int64_t)(ci0 + cc) * P.h_v + h) * 2 * CP + (tid % (2 * CP))];
    };
    // Store chunk cc's raw rows, with window rows before the sequence start
    // (only the first chunk reaches back there).  Rows past its valid tokens
    // repeat the last one (the load is clamped): only padding tokens' v reads
    // them, and a padding token's v cannot reach an output or the state (its
    // b is zero, so its column of T' is zero).
    auto store_raw = [&](int cc, int buf, bool first) {
        const int64_t t0 = s0 + (int64_t)cc * chunk;
        float* dst = s_raw + buf * NRAW * kRows;
#pragma unroll
        for (int it = 0; it < kRawIt; ++it) {
            const int e = tid + it * kThreads;
            const int r = e / kRawVec, cv = (e % kRawVec) * VN;
            if (r < K - 1 + CP) {
                const int64_t p = t0 - (K - 1) + r;
                float x[VN];
#pragma unroll
                for (int i = 0; i < VN; ++i) x[i] = Vec<T>::at(rv[it], i);
                if (first && p < s0) {   // window rows before the sequence start
#pragma unroll
                    for (int i = 0; i < VN; ++i) x[i] = s_win[(K - 1 + (int)(p - s0)) * kRows + cv + i];
                }
#pragma unroll
                for (int i = 0; i < VN; i += 4)
                    *reinterpret_cast<float4*>(dst + r * kRows + cv + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
            }
        }
        if (tid < 2 * CP) s_g[buf * 2 * CP + tid] = rg;
    };
    // conv+SiLU of the block's v channels for chunk cc from s_raw[buf].  All
    // KM taps are applied (weights past conv_k are zero, and the raw rows they
    // meet are finite), so there is no branch between the LDS reads; padding
    // tokens are not masked (see store_raw).
    const int cch = tid % kRows;
    float wv[KM];
#pragma unroll
    for (int m = 0; m < KM; ++m) wv[m] = m < K ? conv_w[(int64_t)(gc0 + cch) * K + m] : 0.f;
    // One channel and TPT consecutive tokens per thread; the outputs are
    // stored channel-major ([channel][token]) so phase 1 reads a lane's four
    // tokens as one vector.
    constexpr int TPT = CP / (kThreads / kRows);
    static_assert(TPT == 2 || TPT == 4, "tokens per thread in the v conv");
    auto conv_v = [&](int buf) {
        const float* src = s_raw + buf * NRAW * kRows;
        float* dst = s_v + buf * CP * kRows;
        const int tt = (tid / kRows) * TPT;
        float xr[TPT + KM - 1];
#pragma unroll
        for (int m = 0; m < TPT + KM - 1; ++m) xr[m] = src[(tt + m) * kRows + cch];
        float y[TPT];
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            float z = 0.f;
#pragma unroll
            for (int m = 0; m < KM; ++m) z = fmaf(wv[m], xr[i + m], z);
            y[i] = silu(z);
        }
        if constexpr (TPT == 4)
            *reinterpret_cast<float4*>(dst + cch * CP + tt) = make_float4(y[0], y[1], y[2], y[3]);
        else
            *reinterpret_cast<float2*>(dst + cch * CP + tt) = make_float2(y[0], y[1]);
    };
    // Publish this wave's state tiles as the B fragment of k-step sw.
    f32x4 st[2];
    auto publish_state = [&]() {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = st[0][i];
            x[4 + i] = st[1][i];
        }
        store_frag(s_stf, sw, lane, split8(x));
    };
    // Lane and element that receive value i of token tile tw, row m16, in the
    // B fragments over tokens (k-step kc = tw/2).
    const int dst_lane = (2 * (tw & 1) + (q4 >> 1)) * 16 + m16;
    const int dst_e0 = 4 * (q4 & 1);
    // Outputs go through a buffer descriptor per chunk, based at the chunk's
    // first row (64-bit address) and bounded at its last valid token, so rows
    // past the sequence end are dropped without a branch and the 32-bit
    // offsets stay inside one chunk however long the sequence is.
    T* out_base = out + (s0 * P.h_v + h) * D + row0;
    const int64_t out_tok = (int64_t)P.h_v * D;       // elements between output rows

    // ---- prologue: state block, old v window, new v window, chunk 0 operands.
    {
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            const float4 x = *reinterpret_cast<const float4*>(
                tile_base + (int64_t)(row0 + m16) * D + (2 * sw + uu) * 16 + q4 * 4);
            st[uu] = f32x4{x.x, x.y, x.z, x.w};
        }
        publish_state();
    }
    if (tid < (K - 1) * kRows) {
        const int r = tid / kRows, c = tid % kRows;
        s_win[r * kRows + c] = Io<T>::load(win, (int64_t)r * C + gc0 + c);
    }
    for (int e = tid; e < 2 * NRAW * kRows; e += kThreads) s_raw[e] = 0.f;
    load_qk(ci0, 1);
    load_qk(ci0, 0);
    load_t(ci0);
    load_p(ci0);
    fetch_raw(0);
    __syncthreads();
    if (tid < (K - 1) * kRows) {   // this workgroup alone owns these channels
        const int r = tid / kRows, c = tid % kRows;
        const int64_t p = s0 + len - (K - 1) + r;
        const float x = p >= s0 ? Io<T>::load(vsrc, p * vstride + c) : s_win[(K - 1 + (int)(p - s0)) * kRows + c];
        Io<T>::store(win, (int64_t)r * C + gc0 + c, x);
    }
    store_raw(0, 0, true);
    __syncthreads();
    conv_v(0);
    // Raw rows are fetched one chunk ahead of their LDS store, which is one
    // phase ahead of their conv.
    fetch_raw(min(1, n_ch - 1));
    __syncthreads();

    for (int cc = 0; cc < n_ch; ++cc) {
        const int buf = cc & 1;
        const bool nxt = cc + 1 < n_ch;
        const int cn = ci0 + min(cc + 1, n_ch - 1);   // next chunk (clamped)
        const int64_t trel = (int64_t)cc * chunk;      // chunk start relative to s0
        // this lane's 4 tokens: gamma = exp(g) and eta = exp(g_last - g)
        const float* gb = s_g + buf * 2 * CP;
        const float4 g4 = *reinterpret_cast<const float4*>(gb + tw * 16 + q4 * 4);
        const float4 e4 = *reinterpret_cast<const float4*>(gb + CP + tw * 16 + q4 * 4);

        // (1) X_K and X_Q for token tile tw, from one read of the state
        // fragments; R = V - diag(gamma) X_K to LDS, XQ = diag(gamma) X_Q in
        // registers until the output.
        f32x4 xq;
        {
            Frag fb[NKS];
            f32x4 acc[NKS], accq[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                fb[ks] = load_frag(s_stf, ks, lane);
                acc[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
                accq[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // the v rows of the tile, requested with the state fragments so
            // that R waits for the MFMAs only (not another LDS round trip)
            const float4 v4 = *reinterpret_cast<const float4*>(s_v + buf * CP * kRows + m16 * CP + tw * 16 + q4 * 4);
            __builtin_amdgcn_sched_barrier(0);
            mma3_n<NKS>(acc, fqk[1], fb);
            mma3_n<NKS>(accq, fqk[0], fb);
            // K^ rows of this token tile into LDS in natural [token][d_k]
            // order (fragment elements 0-3 are d_k 32ks+4q.., 4-7 are +16).
            // Half of them go out while the MFMAs run and half after R: with
            // all 16 writes between the v read and R, the LDS counter (at
            // most 15 outstanding) could only wait for the v read by waiting
            // for every write.
            const auto stage_k = [&](int ks0, int ks1) {
                if (NT * 64 >= kThreads || wave < NT) {   // no branch when every wave has a tile
                    const int kr = tw * 16 + m16, sz = kswz<D>(kr);
                    __bf16* kh = s_kh + kr * KRS;
                    __bf16* kl = s_kl + kr * KRS;
#pragma unroll
                    for (int ks = ks0; ks < ks1; ++ks) {
                        const Frag& f = fqk[1][ks];
                        const int c0 = (ks * 32 + q4 * 4) ^ sz, c1 = (ks * 32 + 16 + q4 * 4) ^ sz;
                        *reinterpret_cast<bf16x4*>(kh + c0) = __builtin_shufflevector(f.hi, f.hi, 0, 1, 2, 3);
                        *reinterpret_cast<bf16x4*>(kh + c1) = __builtin_shufflevector(f.hi, f.hi, 4, 5, 6, 7);
                        *reinterpret_cast<bf16x4*>(kl + c0) = __builtin_shufflevector(f.lo, f.lo, 0, 1, 2, 3);
                        *reinterpret_cast<bf16x4*>(kl + c1) = __builtin_shufflevector(f.lo, f.lo, 4, 5, 6, 7);
                    }
                }
            };
            stage_k(0, NKS / 2);
            f32x4 ak = acc[0];
#pragma unroll
            for (int ks = 1; ks < NKS; ++ks) ak += acc[ks];
            const float r4[4] = {v4.x - g4.x * ak[0], v4.y - g4.y * ak[1],
                                 v4.z - g4.z * ak[2], v4.w - g4.w * ak[3]};
            store_frag4(s_rf, tw >> 1, dst_lane, dst_e0, r4);
            stage_k(NKS / 2, NKS);
            f32x4 aq = accq[0];
#pragma unroll
            for (int ks = 1; ks < NKS; ++ks) aq += accq[ks];
            xq = f32x4{g4.x * aq[0], g4.y * aq[1], g4.z * aq[2], g4.w * aq[3]};
            load_qk(cn, 1);
            load_qk(cn, 0);
        }
        __syncthreads();

        // (2) U = T' R for token tile tw (U and the decayed U to LDS).
        {
            constexpr int NJ = NKC;
            Frag fa[NJ], fb[NJ];
            f32x4 acc[NJ];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                fa[kc] = ftt[kc];
                fb[kc] = load_frag(s_rf, kc, lane);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            mma3_n<NJ>(acc, fa, fb);
            f32x4 uv = acc[0];
#pragma unroll
            for (int kc = 1; kc < NKC; ++kc) uv += acc[kc];
            float u4[4], uu4[4];
            const float el4[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u4[i] = uv[i];
                uu4[i] = uv[i] * el4[i];
            }
            store_frag4(s_uf, tw >> 1, dst_lane, dst_e0, u4);
            store_frag4(s_uuf, tw >> 1, dst_lane, dst_e0, uu4);
            load_t(cn);
        }
        if (nxt) store_raw(cc + 1, buf ^ 1, false);
        __syncthreads();

        // (3) O = XQ + P U for token tile tw, and the state update
        //     S^T <- exp(g_last) S^T + K^T U'' for tiles 2sw, 2sw+1, interleaved.
        {
            constexpr int NJ = 3 * NKC;
            Frag fa[NJ], fb[NJ];
            f32x4 acc[NJ];
            const float dlast = gb[CP - 1];   // gamma of the last token
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const Frag ub = load_frag(s_uf, kc, lane);
                const Frag uub = load_frag(s_uuf, kc, lane);
                fa[kc] = fpp[kc];
                fb[kc] = ub;
                acc[kc] = kc == 0 ? xq : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int uu = 0; uu < 2; ++uu) {
                    // K^T operand of state tile 2sw+uu (rows d_k 16(2sw+uu)+m,
                    // k = tokens 32kc+8q..): transpose reads of the staged K^.
                    // (rows r and r+4 share their swizzle: r % 8 < 4)
                    const int kr = kc * 32 + q4 * 8 + (m16 >> 2), kc0 = (2 * sw + uu) * 16 + 4 * (m16 & 3);
                    const int ko0 = kr * KRS + (kc0 ^ kswz<D>(kr));
                    const int ko1 = (kr + 4) * KRS + (kc0 ^ kswz<D>(kr + 4));
                    Frag kt;
                    kt.hi = __builtin_shufflevector(lds_read_tr(s_kh + ko0), lds_read_tr(s_kh + ko1),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
                    kt.lo = __builtin_shufflevector(lds_read_tr(s_kl + ko0), lds_read_tr(s_kl + ko1),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
                    fa[NKC + uu * NKC + kc] = kt;
                    fb[NKC + uu * NKC + kc] = uub;
                    acc[NKC + uu * NKC + kc] = kc == 0 ? st[uu] * dlast : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
            mma3_n<NJ>(acc, fa, fb);
            f32x4 o = acc[0];
#pragma unroll
            for (int kc = 1; kc < NKC; ++kc) o += acc[kc];
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
                st[uu] = acc[NKC + uu * NKC];
#pragma unroll
                for (int kc = 1; kc < NKC; ++kc) st[uu] += acc[NKC + uu * NKC + kc];
            }
            const int lc = (int)min((int64_t)chunk, len - trel);   // valid rows of the chunk
            const __amdgpu_buffer_rsrc_t out_rs = __builtin_amdgcn_make_buffer_rsrc(
                out_base + trel * out_tok, 0, (int)(((lc - 1) * out_tok + kRows) * sizeof(T)),
                0x00020000);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = tw * 16 + q4 * 4 + i;
                const int off = (int)((t * out_tok + m16) * (int64_t)sizeof(T));
                if constexpr (sizeof(T) == 2)
                    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(o[i]), out_rs, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[i]), out_rs, off, 0, 0);
            }
            publish_state();
            load_p(cn);
        }
        // Checkpoint after a full chunk ending on a multiple of the interval:
        // this block's state rows and its v channels' last conv_k-1 raw rows.
        if (ck.every_chunks > 0 && (cc + 1) % ck.every_chunks == 0 && (cc + 1) * chunk <= len) {
            const int m = (cc + 1) / ck.every_chunks - 1;
            const int cs = m < ck.off[j + 1] - ck.off[j] ? ck.slots[ck.off[j] + m] : -1;
            if (cs >= 0 && cs < P.n_slots) {
                float* cb = P.state + (((int64_t)cs * P.n_layers + layer) * P.h_v + h) * (int64_t)D * D;
                if (wave < NKS) {
#pragma unroll
                    for (int uu = 0; uu < 2; ++uu)
                        *reinterpret_cast<float4*>(cb + (int64_t)(row0 + m16) * D + (2 * wave + uu) * 16 + q4 * 4) =
                            make_float4(st[uu][0], st[uu][1], st[uu][2], st[uu][3]);
                }
                if (tid < (K - 1) * kRows) {
                    const int r = tid / kRows, c = tid % kRows;
                    T* cwin = reinterpret_cast<T*>(P.window) + ((int64_t)cs * P.n_layers + layer) * (int64_t)(K - 1) * C;
                    Io<T>::store(cwin, (int64_t)r * C + gc0 + c, s_raw[buf * NRAW * kRows + (chunk + r) * kRows + c]);
                }
            }
        }
        if (nxt) conv_v(buf ^ 1);
        fetch_raw(min(cc + 2, n_ch - 1));
        prefetch(ci0 + min(cc + 2, n_ch - 1));
        __syncthreads();
    }
    // Keep the prefetch loads alive: OR-ing 0 into the error word changes nothing.
    if ((pf_sink ^ pf_val) == 0x7fc00001u) atomicOr(P.err, 0);

    // ---- store the state block back to the slot.
    if (wave < NKS) {   // waves >= NKS hold copies of tile set NKS-1
#pragma unroll
        for (int uu = 0; uu < 2; ++uu)
            *reinterpret_cast<float4*>(tile_base + (int64_t)(row0 + m16) * D + (2 * wave + uu) * 16 + q4 * 4) =
                make_float4(st[uu][0], st[uu][1], st[uu][2], st[uu][3]);
    }
}

// Factor grids up to this many workgroups run in one round at two per CU.
constexpr int64_t kFactorOneRoundWgs = 512;

// Dynamic LDS of the factor kernel: the largest of its phases (staged rows
// of a pass, the K^ fragments, A and T).
template <int D, int CP, int KC, int NPASS, int NW>
size_t factor_lds_bytes() {
    constexpr int KM = KC > 0 ? KC : kMaxConvK;
    const size_t a = (size_t)(KM - 1 + CP) * (2 * D / NPASS + 4) * sizeof(float);
    const size_t f = (size_t)(CP / 16) * (D / 32) * kFragVecs * 16;
    // A and T per head of a round, then (two groups) the exchanged tiles
    const size_t b = (size_t)(NW / 4) * 2 * CP * (CP + 4) * sizeof(float) +
                     (NW == 8 ? (size_t)2 * (CP / 16) * (CP / 16) * 64 * 16 : 0);
    return std::max(a, std::max(f, b));
}

template <int D, int CP, int KC, typename T>
hipError_t launch_all(const gdn_pool* pool, Ws W, int32_t layer, int32_t n_seq,
                      const int32_t* cu, const int32_t* slot_ids, int total, int chunk, int mc,
                      const void* q, const void* k, const void* v, const float* a, const float* b,
                      const float* conv_w, void* out, Ckpt ck, hipStream_t stream) {
    const PoolView& P = pool->view;
    static std::atomic<uint64_t> factor8_lds{0}, factor1_lds{0}, factor2_lds{0}, scan_lds{0};
    // Factor grids of at most one workgroup per CU run eight waves per
    // workgroup (two value heads side by side); grids that run in one round
    // at two workgroups per CU stage q|k in one pass (the shorter chain per
    // workgroup); larger grids in two, for three workgroups per CU.  Measured
    // at chunk 64 on a Qwen3-Next layer: 16 calls of 512 tokens 866 -> (one
    // pass) us, one 8192-token call 430 -> 416 us and the 16-sequence
    // varlen batch 1537 -> 1442 us with two passes.
    const int64_t nwg = (int64_t)mc * P.h_k;
    const int variant = nwg <= device_cus() ? 8 : nwg <= kFactorOneRoundWgs ? 1 : 2;
    const size_t lf = variant == 8   ? factor_lds_bytes<D, CP, KC, 1, 8>()
                      : variant == 1 ? factor_lds_bytes<D, CP, KC, 1, 4>()
                                     : factor_lds_bytes<D, CP, KC, 2, 4>();
    const size_t ls = ScanLds<D, CP>::bytes;
    hipError_t e = variant == 8   ? allow_dynamic_lds(&prefill_factor_kernel<D, CP, KC, 1, 8, T>, lf, &factor8_lds)
                   : variant == 1 ? allow_dynamic_lds(&prefill_factor_kernel<D, CP, KC, 1, 4, T>, lf, &factor1_lds)
                                  : allow_dynamic_lds(&prefill_factor_kernel<D, CP, KC, 2, 4, T>, lf, &factor2_lds);
    if (e != hipSuccess) return e;
    e = allow_dynamic_lds(&prefill_scan_kernel<D, CP, KC, T>, ls, &scan_lds);
    if (e != hipSuccess) return e;
    // Up to 64 sequences the factor kernel builds the chunk records itself.
    const int fused = n_seq <= kFusedPrepMax ? n_seq : 0;
    if (!fused) {
        hipLaunchKernelGGL(prefill_prep_kernel, dim3(1), dim3(kPrepThreads), 0, stream, P, W, cu,
                           slot_ids, n_seq, total, chunk, mc);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const T* qt = static_cast<const T*>(q);
    const T* kt = static_cast<const T*>(k);
    if (variant == 8)
        hipLaunchKernelGGL((prefill_factor_kernel<D, CP, KC, 1, 8, T>), dim3(mc, P.h_k), dim3(512), lf,
                           stream, P, W, layer, cu, slot_ids, chunk, qt, kt, a, b, conv_w, ck, fused,
                           total, mc);
    else if (variant == 1)
        hipLaunchKernelGGL((prefill_factor_kernel<D, CP, KC, 1, 4, T>), dim3(mc, P.h_k), dim3(256), lf,
                           stream, P, W, layer, cu, slot_ids, chunk, qt, kt, a, b, conv_w, ck, fused,
                           total, mc);
    else
        hipLaunchKernelGGL((prefill_factor_kernel<D, CP, KC, 2, 4, T>), dim3(mc, P.h_k), dim3(256), lf,
                           stream, P, W, layer, cu, slot_ids, chunk, qt, kt, a, b, conv_w, ck, fused,
                           total, mc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_scan_kernel<D, CP, KC, T>), dim3((D / kRows) * P.h_v * n_seq),
                       dim3(kThreads), ls, stream, P, W, layer, chunk, static_cast<const T*>(v),
                       conv_w, static_cast<T*>(out), ck);
    return hipGetLastError();
}

template <int D, int KC, typename T>
hipError_t launch_dk(const gdn_pool* pool, Ws W, int32_t layer, int32_t n_seq, const int32_t* cu,
                     const int32_t* slot_ids, int total, int chunk, int mc, const void* q,
                     const void* k, const void* v, const float* a, const float* b,
                     const float* conv_w, void* out, Ckpt ck, hipStream_t stream) {
    if (chunk == 64)
        return launch_all<D, 64, KC, T>(pool, W, layer, n_seq, cu, slot_ids, total, chunk, mc, q, k,
                                        v, a, b, conv_w, out, ck, stream);
    return launch_all<D, 32, KC, T>(pool, W, layer, n_seq, cu, slot_ids, total, chunk, mc, q, k, v,
                                    a, b, conv_w, out, ck, stream);
}

// conv_k = 4 (the common width) gets kernels with the taps fixed at compile
// time; other widths use the runtime-width kernels.
template <int D, typename T>
hipError_t launch_d(const gdn_pool* pool, Ws W, int32_t layer, int32_t n_seq, const int32_t* cu,
                    const int32_t* slot_ids, int total, int chunk, int mc, const void* q,
                    const void* k, const void* v, const float* a, const float* b,
                    const float* conv_w, void* out, Ckpt ck, hipStream_t stream) {
    if (pool->view.conv_k == 4)
        return launch_dk<D, 4, T>(pool, W, layer, n_seq, cu, slot_ids, total, chunk, mc, q, k, v, a,
                                  b, conv_w, out, ck, stream);
    return launch_dk<D, 0, T>(pool, W, layer, n_seq, cu, slot_ids, total, chunk, mc, q, k, v, a, b,
                              conv_w, out, ck, stream);
}

// Device-resident prefill workspace for callers that cannot allocate
// (gdn_prefill_chunked_static).  Every device the library runs on holds one
// until the process ends.  Its name is only a host-side handle: the kernels
// get the per-device address that hipGetSymbolAddress returns.
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t prefill_static_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        // first call on this device (the device is current): resolve the
        // array's address on it once
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

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
                          void* out, void* workspace, Ckpt ck, hipStream_t stream) {
    const PoolView& P = pool->view;
    size_t bytes = 0;
    Ws W = carve(workspace, P, n_seq, total_tokens, chunk, &bytes);
    const int64_t mc = max_chunks(n_seq, total_tokens, chunk);
    if (mc > INT32_MAX || n_seq > 65535) return hipErrorNotSupported;
    if (P.h_v / P.h_k > 4) return hipErrorNotSupported;   // value heads per group kept in LDS
    // One chunk of output rows is addressed with 32-bit offsets.
    if ((int64_t)64 * P.h_v * P.d * pool->io_size >= INT32_MAX) return hipErrorNotSupported;
    const bool bf = pool->desc.io_dtype == GDN_BF16;
    const int total = (int)total_tokens, m = (int)mc;
    switch (P.d) {
#define GDN_CASE(DD)                                                                             \
    case DD:                                                                                     \
        return bf ? launch_d<DD, uint16_t>(pool, W, layer, n_seq, cu_seqlens, slot_ids, total,   \
                                           chunk, m, q, k, v, a, b, conv_w, out, ck, stream)     \
                  : launch_d<DD, float>(pool, W, layer, n_seq, cu_seqlens, slot_ids, total,      \
                                        chunk, m, q, k, v, a, b, conv_w, out, ck, stream);
        GDN_CASE(32)
        GDN_CASE(64)
        GDN_CASE(128)
#undef GDN_CASE
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace gdn
