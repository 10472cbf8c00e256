// Split-precision bf16 MFMA helpers (gfx950), shared by the kernels that run
// fp32 contractions on the matrix cores.  Every fp32 operand x is split as
// hi = bf16(x), lo = bf16(x - hi) and a product is taken as
// hi*hi + hi*lo + lo*hi with fp32 accumulation, which keeps it within a few
// fp32 ulps of the fp32 product (lo*lo is below fp32 rounding).
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One lane's share of a 16x16x32 bf16 MFMA operand, split as hi + lo.
// Lane l = 16 q + m of an A operand holds row m, k = 8q..8q+7; of a B operand
// column m, k = 8q..8q+7; the fp32 result holds rows 4q..4q+3 of column m.
struct Frag {
    bf16x8 hi, lo;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Split of two floats: hi = their bf16 pair (one packed conversion), the
// fp32 values of the two halves by a shift and a mask, lo = the packed bf16
// of the two exact differences.  Bitwise the same as converting each value
// on its own, in six instructions per pair instead of eight.
__device__ __forceinline__ void split2(float a, float b, bf16x2& hi, bf16x2& lo) {
    hi = bf16x2{(__bf16)a, (__bf16)b};
    const uint32_t h = __builtin_bit_cast(uint32_t, hi);
    const float ha = __uint_as_float(h << 16), hb = __uint_as_float(h & 0xffff0000u);
    lo = bf16x2{(__bf16)(a - ha), (__bf16)(b - hb)};
}

__device__ __forceinline__ Frag split8(const float* x) {
    Frag r;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
        bf16x2 h, l;
        split2(x[j], x[j + 1], h, l);
        r.hi[j] = h[0];
        r.hi[j + 1] = h[1];
        r.lo[j] = l[0];
        r.lo[j + 1] = l[1];
    }
    return r;
}

// acc += A * B for one 16x16x32 tile.
__device__ __forceinline__ f32x4 mma3(f32x4 acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    return acc;
}

// acc[j] += a[j] * b[j] for N independent tiles, with the three hi/lo products
// of all tiles interleaved so that consecutive MFMAs never depend on each
// other (a dependent MFMA would wait for the previous one to drain).
template <int N>
__device__ __forceinline__ void mma3_n(f32x4* acc, const Frag* a, const Frag* b) {
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j].lo, b[j].hi, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j].hi, b[j].lo, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j].hi, b[j].hi, acc[j], 0, 0, 0);
}

// Fragment buffers: [fragment][hi | lo][64 lanes] of 16-byte vectors, 2 KiB
// per fragment, so a wave reads or writes one half in one coalesced 1 KiB.
constexpr int kFragVecs = 128;   // bf16x8 per fragment

__device__ __forceinline__ void store_frag(bf16x8* base, int f, int lane, const Frag& x) {
    base[f * kFragVecs + lane] = x.hi;
    base[f * kFragVecs + 64 + lane] = x.lo;
}
// The same with non-temporal stores, for fragments written to global memory
// that the writing kernel does not read again.
__device__ __forceinline__ void store_frag_nt(bf16x8* base, int f, int lane, const Frag& x) {
    __builtin_nontemporal_store(x.hi, base + f * kFragVecs + lane);
    __builtin_nontemporal_store(x.lo, base + f * kFragVecs + 64 + lane);
}
__device__ __forceinline__ Frag load_frag(const bf16x8* base, int f, int lane) {
    Frag x;
    x.hi = base[f * kFragVecs + lane];
    x.lo = base[f * kFragVecs + 64 + lane];
    return x;
}

// Eight floats from two 16-byte aligned groups of four.
__device__ __forceinline__ void ld4x2(float* dst, const float* lo, const float* hi) {
    const float4 x0 = *reinterpret_cast<const float4*>(lo);
    const float4 x1 = *reinterpret_cast<const float4*>(hi);
    dst[0] = x0.x; dst[1] = x0.y; dst[2] = x0.z; dst[3] = x0.w;
    dst[4] = x1.x; dst[5] = x1.y; dst[6] = x1.z; dst[7] = x1.w;
}

__device__ __forceinline__ void ld8(float* dst, const float* src) { ld4x2(dst, src, src + 4); }

}  // namespace gdn
