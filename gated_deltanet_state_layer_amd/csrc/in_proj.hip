// Input projection in front of the conv: y = x W^T over the hidden size, for
// a batch of tokens, written straight into the raw q, k, v the other calls
// take and the two gates a = exp(-softplus(y_a)) = 1 / (1 + e^y_a) and
// b = sigmoid(y_b) ("baseRT issue #31", section "Why this looks tractable":
// an input-projection kernel sits beside the conv in the layer's kernels).
// W's rows are the output channels, in the order q heads | k heads | v heads
// | h_v a logits | h_v b logits; x and W are bf16, products are exact in fp32
// and accumulate in fp32 on the bf16 matrix cores.
//
// Up to 64 tokens: the skinny kernel below.  From 512 tokens (when the hidden
// dimension is not split): the 256 x 256 tile kernel, plus the skinny kernel
// for the channels past its last full 256-channel column.  Otherwise the
// gemm kernel: grid (N/128, M/128, ksplit), 4 waves, a 128 x 128 output tile
// per workgroup; k-blocks of 64 go through two LDS stages, filled one block
// ahead by 16-byte buffer loads that write LDS directly and whose descriptors
// return zeros past the ragged ends.
// With few tokens the hidden dimension is split over ksplit workgroups so
// that enough weight bytes are in flight; a second kernel adds the partial
// sums.  Otherwise the gemm kernel writes the outputs itself.
#include <algorithm>

#include "gdn_common.h"
#include "mfma_split.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kRsrcWord3 = 0x00020000;
// An offset past every descriptor used here: the calls accept x and W only
// below INT32_MAX - 256 * hidden bytes (hidden >= 32), so below 0x7fffe000.
constexpr int kOffOOB = 0x7ffffff0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcWord3);
}

struct ProjOut {
    void *q, *k, *v;
    float *a, *b;
    int hkd, hvd, c_conv, h_v, n_out;
    int vec8;   // q, k, v 16-byte aligned and hkd, hvd, c_conv multiples of 8
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

// Outputs n .. n+7 of token m (n a multiple of 8).  With vec8, eight
// channels below c_conv lie in one of q, k, v and go out as one 16-byte
// (bf16) or two 16-byte (fp32) stores; otherwise (and for the gates) one by
// one, skipping channels past n_out.
template <typename T>
__device__ __forceinline__ void put8(const ProjOut& o, int64_t m, int n, const float* y) {
    if (o.vec8 && n < o.c_conv) {
        T* dst;
        int64_t off;
        if (n < o.hkd) {
            dst = static_cast<T*>(o.q);
            off = m * o.hkd + n;
        } else if (n < 2 * o.hkd) {
            dst = static_cast<T*>(o.k);
            off = m * o.hkd + n - o.hkd;
        } else {
            dst = static_cast<T*>(o.v);
            off = m * o.hvd + n - 2 * o.hkd;
        }
        if constexpr (sizeof(T) == 2) {
            uint4 pk;
            pk.x = f32_to_bf16(y[0]) | (uint32_t)f32_to_bf16(y[1]) << 16;
            pk.y = f32_to_bf16(y[2]) | (uint32_t)f32_to_bf16(y[3]) << 16;
            pk.z = f32_to_bf16(y[4]) | (uint32_t)f32_to_bf16(y[5]) << 16;
            pk.w = f32_to_bf16(y[6]) | (uint32_t)f32_to_bf16(y[7]) << 16;
            *reinterpret_cast<uint4*>(dst + off) = pk;
        } else {
            *reinterpret_cast<float4*>(dst + off) = make_float4(y[0], y[1], y[2], y[3]);
            *reinterpret_cast<float4*>(dst + off + 4) = make_float4(y[4], y[5], y[6], y[7]);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (n + i < o.n_out) put<T>(o, m, n + i, y[i]);
}

// 128 x 128 output tile per workgroup (wave (wm, wn) owns a 64 x 64
// quadrant: 4 x 4 MFMA tiles), k-blocks of 64 in two LDS stages of 32 KiB:
// the loads of block kb+1 go out while the waves multiply block kb, straight
// into LDS, with no staging registers and one barrier per block.  Against a
// ring of three stages of k 32 this took 96 / 256 / 511 tokens (hidden 2048)
// from 23.0 / 30.8 / 45.3 to 21.9 / 27.9 / 38.9 us, same box.
constexpr int BM = 128, BN = 128, BK = 32;

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void in_proj_gemm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int M, int H, ProjOut o,
    float* __restrict__ part, int blocks_per_split) {
    // Two stages of (128 x rows + 128 W rows) x 64 k, 128 bytes per row,
    // filled by loads that write LDS directly, as in the wide kernel below.
    constexpr int KB = 64;                           // k per stage
    constexpr int kStage = (BM + BN) * KB;           // bf16 per stage
    __shared__ __align__(16) uint16_t sa[2 * kStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m16 = lane & 15, q4 = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int N = o.n_out;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    // this split's k range, [k_begin, k_end), in steps of KB
    const int k_begin = blockIdx.z * blocks_per_split * BK;
    const int k_end = min(H, k_begin + blocks_per_split * BK);
    const int nkb = k_end > k_begin ? (k_end - k_begin + KB - 1) / KB : 0;
    const auto x_rs = buf_rsrc(x, M * H * 2), w_rs = buf_rsrc(w, N * H * 2);
    // Each wave fills 32 x rows and 32 W rows per stage, 8 rows of 128 bytes
    // per load: lane l writes row l / 8, slot l % 8, and slot s of row r
    // holds the k-chunk s ^ ((r / 2) % 8).  Rows past M or N, and chunks past
    // the split's end, read zeros (offsets past the descriptors).
    const int lrow = lane >> 3, lslot = lane & 7;
    int gx[4], gw[4], kc[4];
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
        const int r = wave * 32 + i2 * 8 + lrow;
        kc[i2] = lslot ^ ((4 * i2 + (lrow >> 1)) & 7);
        gx[i2] = m0 + r < M ? ((m0 + r) * H + kc[i2] * 8) * 2 : kOffOOB;
        gw[i2] = n0 + r < N ? ((n0 + r) * H + kc[i2] * 8) * 2 : kOffOOB;
    }
    using lds_ptr = __attribute__((address_space(3))) void*;
    auto issue = [&](int kb, int st) {
        uint16_t* base = sa + st * kStage;
        const int k0 = k_begin + kb * KB;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            const bool in_k = k0 + kc[i2] * 8 < k_end;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                x_rs, (lds_ptr)(base + (wave * 32 + i2 * 8) * KB), 16,
                gx[i2] == kOffOOB || !in_k ? kOffOOB : gx[i2] + k0 * 2, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                w_rs, (lds_ptr)(base + (BM + wave * 32 + i2 * 8) * KB), 16,
                gw[i2] == kOffOOB || !in_k ? kOffOOB : gw[i2] + k0 * 2, 0, 0, 0);
        }
    };
    const int rkey = (m16 >> 1) & 7;
    f32x4 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nkb > 0) issue(0, 0);
    for (int kb = 0; kb < nkb; ++kb) {
        // this thread's loads of block kb are done, then every thread's are,
        // and every wave has finished reading the stage block kb + 1 goes to
        __builtin_amdgcn_s_waitcnt(0x0f70);                      // vmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        if (kb + 1 < nkb) issue(kb + 1, (kb + 1) & 1);
        const uint16_t* sx = sa + (kb & 1) * kStage;
        const uint16_t* sw = sx + BM * KB;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const int so = 8 * ((kh * 4 + q4) ^ rkey);
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                fa[mt] = *reinterpret_cast<const bf16x8*>(&sx[(wm * 64 + mt * 16 + m16) * KB + so]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                fb[nt] = *reinterpret_cast<const bf16x8*>(&sw[(wn * 64 + nt * 16 + m16) * KB + so]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mt], fb[nt], acc[mt][nt], 0, 0, 0);
        }
    }
    // lane holds y[m0 + 64 wm + 16 mt + 4 q + j][n0 + 64 wn + 16 nt + m16]
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int n = n0 + wn * 64 + nt * 16 + m16;
        if (n >= N) continue;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = m0 + wm * 64 + mt * 16 + q4 * 4 + j;
                if (m >= M) continue;
                if (part) part[((int64_t)blockIdx.z * M + m) * N + n] = acc[mt][nt][j];
                else put<T>(o, m, n, acc[mt][nt][j]);
            }
    }
}

// Many tokens: a 256 x 256 output tile per workgroup of 8 waves, wave (wm, wn)
// owning a 128 x 64 block (8 x 4 MFMA tiles), so each wave reads 384 bytes of
// LDS operands per MFMA instead of the 512 of a 64 x 64 block.  k-blocks of
// 64 (64 MFMAs per wave between barriers) go through two LDS stages of
// 64 KiB, written by buffer loads that store straight into LDS (no staging
// registers), issued one block ahead; one barrier per block.  One workgroup
// per CU (128 KiB of LDS), two waves per SIMD.  Measured at 8192 tokens
// (hidden 2048), same-box A/Bs: against double-buffered register staging of
// a 256 x 128 tile (each thread loading its share of block kb+1 into
// registers while the waves multiply block kb, then writing it to LDS), the
// direct loads (three stages of k 32) took the call from 369-381 to
// 336-343 us; the 256 x 256 tile (a quarter fewer operand bytes per MFMA
// from L2) from 341-362 to 324-341 us (a fourth stage: no faster); k-blocks
// of 64 in two stages (half the barriers) from 323-332 to 298-303 us.  It
// covers the full 256-channel columns only: the channels past the last of
// them (the 64 gate logits when the q|k|v channels are a multiple of 256) go
// to the skinny kernel below in a second short launch.  A partial column
// would add a fifth round of tiles at 8192 tokens for 1/128 of the work.
constexpr int BM2 = 256, BN2 = 256;
constexpr int kWideThreads = 512;

template <typename T>
__global__ __launch_bounds__(kWideThreads, 1) void in_proj_wide_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int M, int H, ProjOut o,
    int n_tn) {
    // Two stages of (256 x rows + 256 W rows) x 64 k, 128 bytes per row,
    // filled by loads that write LDS directly (no registers in between).
    // Those loads count on vmcnt until their data is in LDS; the waits in the
    // loop below are explicit, since nothing else orders the LDS reads after
    // them.
    constexpr int KB = 64;                           // k per stage
    constexpr int kStage = (BM2 + BN2) * KB;          // bf16 per stage
    __shared__ __align__(16) uint16_t sa[2 * kStage];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m16 = lane & 15, q4 = lane >> 4;
    const int wm = wave >> 2, wn = wave & 3;
    const int N = o.n_out;
    const int n_tm = (M + BM2 - 1) / BM2;
    // Tile order: column-major (consecutive ids share their W rows).  A
    // banded order that gives each XCD a compact 8 x 8 group of tiles was
    // measured no faster with a 256 x 128 tile (385 vs 379 us at 8192 tokens).
    const int t = blockIdx.x;
    if (t >= n_tm * n_tn) return;
    const int tm = t % n_tm, tn = t / n_tm;
    const int m0 = tm * BM2, n0 = tn * BN2;
    const int nblk = (H + KB - 1) / KB;
    const auto x_rs = buf_rsrc(x, M * H * 2), w_rs = buf_rsrc(w, N * H * 2);
    // One load instruction fills 8 rows of 128 bytes (1 KiB): lane l writes
    // bytes 16 l .. 16 l + 15 after the wave-uniform base, i.e. row l / 8,
    // slot l % 8.  Slot s of row r holds the k-chunk s ^ ((r / 2) % 8), so
    // that the 16 rows of an MFMA fragment read hit 16 different bank
    // groups.  Rows past M or N, and chunks past H (hidden sizes that are odd
    // multiples of 32), read zeros (offset past the descriptor).
    const int lrow = lane >> 3, lslot = lane & 7;
    int gx[4], gw[4], kc[4];
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
        const int r = wave * 32 + i2 * 8 + lrow;
        kc[i2] = lslot ^ ((4 * i2 + (lrow >> 1)) & 7);
        gx[i2] = m0 + r < M ? ((m0 + r) * H + kc[i2] * 8) * 2 : kOffOOB;
        gw[i2] = n0 + r < N ? ((n0 + r) * H + kc[i2] * 8) * 2 : kOffOOB;
    }
    using lds_ptr = __attribute__((address_space(3))) void*;
    auto issue = [&](int kb, int st) {
        uint16_t* base = sa + st * kStage;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            const bool in_k = kb * KB + kc[i2] * 8 < H;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                x_rs, (lds_ptr)(base + (wave * 32 + i2 * 8) * KB), 16,
                gx[i2] == kOffOOB || !in_k ? kOffOOB : gx[i2] + kb * KB * 2, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                w_rs, (lds_ptr)(base + (BM2 + wave * 32 + i2 * 8) * KB), 16,
                gw[i2] == kOffOOB || !in_k ? kOffOOB : gw[i2] + kb * KB * 2, 0, 0, 0);
        }
    };
    const int rkey = (m16 >> 1) & 7;
    f32x4 acc[8][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    issue(0, 0);
    for (int kb = 0; kb < nblk; ++kb) {
        // this thread's loads of block kb are done, then every thread's are,
        // and every wave has finished reading the stage block kb + 1 goes to
        __builtin_amdgcn_s_waitcnt(0x0f70);                      // vmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        if (kb + 1 < nblk) issue(kb + 1, (kb + 1) & 1);
        const uint16_t* sx = sa + (kb & 1) * kStage;
        const uint16_t* sw = sx + BM2 * KB;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const int so = 8 * ((kh * 4 + q4) ^ rkey);
            bf16x8 fa[8], fb[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                fb[nt] = *reinterpret_cast<const bf16x8*>(&sw[(wn * 64 + nt * 16 + m16) * KB + so]);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                fa[mt] = *reinterpret_cast<const bf16x8*>(&sx[(wm * 128 + mt * 16 + m16) * KB + so]);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[mt], fb[nt], acc[mt][nt], 0, 0, 0);
        }
    }
    __syncthreads();   // every wave is done with the operand stages
    // Epilogue through LDS: lane (m16, q4) holds rows 16 mt + 4 q4 + j of
    // column 16 nt + m16 of the wave's 128 x 64 block, so stores straight from
    // the accumulators write 2- or 4-byte pieces.  Each wave instead writes 32
    // of its rows at a time to a private fp32 buffer in the (now free) operand
    // LDS and reads them back as eight consecutive channels per lane for
    // put8.  The last k-block's barrier has passed, so no wave still reads
    // sa/sb; each wave touches only its own buffer, so no barrier is needed.
    // lane holds y[m0 + 128 wm + 16 mt + 4 q + j][n0 + 64 wn + 16 nt + m16]
    constexpr int ER = 32, ELD = 64 + 4;   // rows per pass; padded row (floats)
    static_assert(8 * ER * ELD * sizeof(float) <= sizeof(sa), "epilogue buffer fits in sa");
    float* eb = reinterpret_cast<float*>(&sa[0]) + wave * ER * ELD;
#pragma unroll
    for (int pass = 0; pass < 128 / ER; ++pass) {
#pragma unroll
        for (int mh = 0; mh < ER / 16; ++mh)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    eb[(mh * 16 + q4 * 4 + j) * ELD + nt * 16 + m16] = acc[pass * (ER / 16) + mh][nt][j];
        // read back: 32 rows x 8 groups of 8 channels = 4 groups per lane
#pragma unroll
        for (int it = 0; it < ER * 8 / 64; ++it) {
            const int gidx = lane + it * 64, r = gidx >> 3, c8 = (gidx & 7) * 8;
            const float4 p0 = *reinterpret_cast<const float4*>(eb + r * ELD + c8);
            const float4 p1 = *reinterpret_cast<const float4*>(eb + r * ELD + c8 + 4);
            const float y[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            const int m = m0 + wm * 128 + pass * ER + r, n = n0 + wn * 64 + c8;
            if (m < M && n < N) put8<T>(o, m, n, y);
        }
    }
}

// Few tokens (M <= 64): the weight stream is the whole cost.  One workgroup
// of 8 waves per 64 output channels and 64 tokens (grid y; also used, with 32
// tokens per workgroup when each wave has 8 k-steps, for the channels past
// the last full column of the 256-token-tile kernel); wave w multiplies the
// full 64 x 64 tile over its eighth of the hidden dimension, operands straight from memory into
// MFMA registers (16 bytes per lane, one step ahead), and the eight partial
// tiles are added in LDS before the fused epilogue.  No partial sums leave
// the chip and there is no second launch.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyStages = 4;   // k-steps of operand loads in flight per wave
constexpr int kSkinnyThreads = 64 * kSkinnyWaves;
constexpr size_t kSkinnyLds = (size_t)kSkinnyWaves * 64 * 64 * sizeof(float);

// NS > 0: each wave's k-step count fixed at compile time (the loop below is
// then straight-line code with exact waits); 0: any count.  TMT: 16-token
// tiles per workgroup, 4 (64 tokens) or 2 (32 tokens: half the registers and
// LDS, so two workgroups fit per CU; three k-steps in flight to stay within
// 128 registers).
template <typename T, int NS, int TMT = 4>
__global__ __launch_bounds__(kSkinnyThreads, TMT < 4 ? 4 : 1) void in_proj_skinny_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int M, int H, ProjOut o,
    int c0) {
    constexpr int kStg = TMT < 4 ? 3 : kSkinnyStages;
    extern __shared__ __align__(16) float red[];     // [8 waves][16 TMT tokens][64 channels]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m16 = lane & 15, q4 = lane >> 4;
    const int N = o.n_out, n0 = c0 + blockIdx.x * 64, m0 = blockIdx.y * 16 * TMT;
    const int nsteps = H / 32, per = (nsteps + kSkinnyWaves - 1) / kSkinnyWaves;
    const int s_begin = wave * per, s_end = min(nsteps, s_begin + per);
    const auto x_rs = buf_rsrc(x, M * H * 2), w_rs = buf_rsrc(w, N * H * 2);
    int xo[TMT], wo[4];
#pragma unroll
    for (int t = 0; t < TMT; ++t) xo[t] = ((m0 + t * 16 + m16) * H) * 2 + q4 * 16;    // tokens past M read zeros
#pragma unroll
    for (int t = 0; t < 4; ++t) wo[t] = ((n0 + t * 16 + m16) * H) * 2 + q4 * 16;    // channels past N read zeros
    auto fetch = [&](int st, bf16x8* xf, bf16x8* wf) {
        const bool ok = st < s_end;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < TMT)
                xf[t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(x_rs, ok ? xo[t] + st * 64 : kOffOOB, 0, 0));
            wf[t] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(w_rs, ok ? wo[t] + st * 64 : kOffOOB, 0, 0));
        }
    };
    f32x4 acc[TMT][4];
#pragma unroll
    for (int mt = 0; mt < TMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Up to kSkinnyStages k-steps of loads in flight per wave: a step's MFMAs
    // take ~0.1 us, the loads ~1-2 us, so one step of prefetch would leave
    // every step waiting a whole memory latency.  Each stage's registers are
    // refilled right after its MFMAs.  Steps past the wave's range load zeros
    // (no memory access).
    bf16x8 xs[kStg][4], ws[kStg][4];
    auto mma_stage = [&](int i) {
#pragma unroll
        for (int mt = 0; mt < TMT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xs[i][mt], ws[i][nt], acc[mt][nt], 0, 0, 0);
    };
    if constexpr (NS > 0) {
        // Straight-line pipeline.  The scheduling barriers keep each stage's
        // loads where they are written: left alone, the scheduler sinks them
        // next to their MFMAs to save registers, and every step waits again.
#pragma unroll
        for (int i = 0; i < kStg && i < NS; ++i) fetch(s_begin + i, xs[i], ws[i]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            mma_stage(j % kStg);
            if (j + kStg < NS) fetch(s_begin + j + kStg, xs[j % kStg], ws[j % kStg]);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        // Any step count: two stages, one step ahead.
        fetch(s_begin, xs[0], ws[0]);
        for (int st = s_begin; st < s_end; st += 2) {
            fetch(st + 1, xs[1], ws[1]);
            mma_stage(0);
            fetch(st + 2, xs[0], ws[0]);
            mma_stage(1);   // zeros past the range
        }
    }
    // lane holds y[m0 + 16 mt + 4 q + j][n0 + 16 nt + m16]
    float* mine = red + wave * TMT * 16 * 64;
#pragma unroll
    for (int mt = 0; mt < TMT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int j = 0; j < 4; ++j) mine[(mt * 16 + q4 * 4 + j) * 64 + nt * 16 + m16] = acc[mt][nt][j];
    __syncthreads();
    for (int idx = tid; idx < TMT * 16 * 64; idx += kSkinnyThreads) {
        const int m = m0 + (idx >> 6), n = n0 + (idx & 63);
        if (m >= M || n >= N) continue;
        float y = 0.f;
#pragma unroll
        for (int ww = 0; ww < kSkinnyWaves; ++ww) y += red[ww * TMT * 16 * 64 + idx];
        put<T>(o, m, n, y);
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

// From this many tokens (and no split of the hidden dimension) the 256 x 256
// tile kernel runs.
constexpr int64_t kWideMinTokens = 512;

// Split of the hidden dimension for M tokens: enough workgroups to keep the
// weight stream busy, at least 4 k-blocks of 32 per split.
int in_proj_ksplit(const gdn_pool* pool, int64_t M, int32_t H) {
    if (M <= 64) return 1;   // the skinny kernel
    const int N = pool->view.c_conv + 2 * pool->view.h_v;
    const int64_t tiles = (int64_t)((N + BN - 1) / BN) * ((M + BM - 1) / BM);
    int ks = (int)std::min<int64_t>(16, std::max<int64_t>(1, 512 / std::max<int64_t>(tiles, 1)));
    ks = std::min(ks, std::max(1, H / BK / 4));
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
    const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const int hkd = P.h_k * P.d, hvd = P.h_v * P.d;
    ProjOut o{q, k, v, a, b, hkd, hvd, P.c_conv, P.h_v, P.c_conv + 2 * P.h_v,
              al16(q) && al16(k) && al16(v) && hkd % 8 == 0 && hvd % 8 == 0 && P.c_conv % 8 == 0};
    const auto* xs = static_cast<const uint16_t*>(x);
    const auto* ws = static_cast<const uint16_t*>(w);
    const bool bf = pool->desc.io_dtype == GDN_BF16;
    // Skinny kernel over channels [c0, n_out) and all M tokens, 64 x 64 per workgroup.
    auto skinny = [&](int c0) -> hipError_t {
        // more than 64 KiB of dynamic LDS: enabled once per kernel and device
        static std::atomic<uint64_t> lds_bf{0}, lds_f{0};
        static std::atomic<uint64_t> lds_bf8{0}, lds_f8{0};
        const bool ns8 = (H / 32 + kSkinnyWaves - 1) / kSkinnyWaves == 8;   // e.g. hidden 2048
        const hipError_t e =
            bf ? (ns8 ? allow_dynamic_lds(&in_proj_skinny_kernel<uint16_t, 8>, kSkinnyLds, &lds_bf8)
                      : allow_dynamic_lds(&in_proj_skinny_kernel<uint16_t, 0>, kSkinnyLds, &lds_bf))
               : (ns8 ? allow_dynamic_lds(&in_proj_skinny_kernel<float, 8>, kSkinnyLds, &lds_f8)
                      : allow_dynamic_lds(&in_proj_skinny_kernel<float, 0>, kSkinnyLds, &lds_f));
        if (e != hipSuccess) return e;
        const dim3 grid((o.n_out - c0 + 63) / 64, (unsigned)((M + 63) / 64));
        if (bf && ns8)
            hipLaunchKernelGGL((in_proj_skinny_kernel<uint16_t, 8>), grid, dim3(kSkinnyThreads), kSkinnyLds,
                               stream, xs, ws, (int)M, H, o, c0);
        else if (bf)
            hipLaunchKernelGGL((in_proj_skinny_kernel<uint16_t, 0>), grid, dim3(kSkinnyThreads), kSkinnyLds,
                               stream, xs, ws, (int)M, H, o, c0);
        else if (ns8)
            hipLaunchKernelGGL((in_proj_skinny_kernel<float, 8>), grid, dim3(kSkinnyThreads), kSkinnyLds,
                               stream, xs, ws, (int)M, H, o, c0);
        else
            hipLaunchKernelGGL((in_proj_skinny_kernel<float, 0>), grid, dim3(kSkinnyThreads), kSkinnyLds,
                               stream, xs, ws, (int)M, H, o, c0);
        return hipGetLastError();
    };
    if (M <= 64) return skinny(0);
    const int ks = in_proj_ksplit(pool, M, H);
    const int n_full = o.n_out / BN2;   // full 256-channel columns
    if (ks == 1 && M >= kWideMinTokens && n_full > 0) {
        const int tiles = (int)((M + BM2 - 1) / BM2) * n_full;
        const dim3 grid((unsigned)tiles);
        if (bf)
            hipLaunchKernelGGL(in_proj_wide_kernel<uint16_t>, grid, dim3(kWideThreads), 0, stream, xs, ws,
                               (int)M, H, o, n_full);
        else
            hipLaunchKernelGGL(in_proj_wide_kernel<float>, grid, dim3(kWideThreads), 0, stream, xs, ws,
                               (int)M, H, o, n_full);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || n_full * BN2 == o.n_out) return e;
        if ((H / 32 + kSkinnyWaves - 1) / kSkinnyWaves == 8) {
            // The strip past the last full column with 32 tokens per
            // workgroup: at 8192 tokens 256 workgroups instead of 128, each
            // streaming half as much of x (21.6 -> ~14 us for the 64 gate
            // channels at hidden 2048).
            const int c0 = n_full * BN2;
            const dim3 g2((o.n_out - c0 + 63) / 64, (unsigned)((M + 31) / 32));
            const size_t lds = (size_t)kSkinnyWaves * 32 * 64 * sizeof(float);
            if (bf)
                hipLaunchKernelGGL((in_proj_skinny_kernel<uint16_t, 8, 2>), g2, dim3(kSkinnyThreads), lds,
                                   stream, xs, ws, (int)M, H, o, c0);
            else
                hipLaunchKernelGGL((in_proj_skinny_kernel<float, 8, 2>), g2, dim3(kSkinnyThreads), lds,
                                   stream, xs, ws, (int)M, H, o, c0);
            return hipGetLastError();
        }
        return skinny(n_full * BN2);
    }
    const int nblk = H / BK, per = (nblk + ks - 1) / ks;
    float* part = ks > 1 ? static_cast<float*>(workspace) : nullptr;
    const dim3 grid((o.n_out + BN - 1) / BN, (unsigned)((M + BM - 1) / BM), ks);
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
