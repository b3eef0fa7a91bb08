// Device helpers shared by the Lighthouse kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lh.h"

namespace lh {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Two fp32 values to two bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 values to two fp16 (round to nearest even, v_cvt_pk_f16_f32; beyond
// the fp16 range the result is +-inf), packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void unpack_f16x2(uint32_t u, float &lo, float &hi)
{
    const f16x2_t v = __builtin_bit_cast(f16x2_t, u);
    lo = (float)v[0];
    hi = (float)v[1];
}

// 8 fp32 values as 8 fp16 (one 16-byte word).
__device__ __forceinline__ uint4 pack8_f16(const float (&x)[8])
{
    return make_uint4(pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]), pack_f16x2(x[4], x[5]), pack_f16x2(x[6], x[7]));
}

__device__ __forceinline__ void unpack8_f16(uint4 u, float (&x)[8])
{
    unpack_f16x2(u.x, x[0], x[1]);
    unpack_f16x2(u.y, x[2], x[3]);
    unpack_f16x2(u.z, x[4], x[5]);
    unpack_f16x2(u.w, x[6], x[7]);
}

// x = hi + lo with hi = fp16(x) and lo = fp16(x - hi): about 22 significant bits.
__device__ __forceinline__ void split8_f16(const float (&x)[8], uint4 &hi, uint4 &lo)
{
    hi = pack8_f16(x);
    float h[8], r[8];
    unpack8_f16(hi, h);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        r[e] = x[e] - h[e];
    lo = pack8_f16(r);
}

// ---------------------------------------------------------------- 8-element row pieces
// A "piece" is 8 consecutive elements of a row, converted to fp32.
__device__ __forceinline__ void load8(const uint16_t *p, float (&x)[8])
{
    uint4 u = *reinterpret_cast<const uint4 *>(p);
    x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xffff0000u);
    x[4] = __uint_as_float(u.z << 16); x[5] = __uint_as_float(u.z & 0xffff0000u);
    x[6] = __uint_as_float(u.w << 16); x[7] = __uint_as_float(u.w & 0xffff0000u);
}

__device__ __forceinline__ void load8(const float *p, float (&x)[8])
{
    float4 a = reinterpret_cast<const float4 *>(p)[0];
    float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void store8(uint16_t *p, const float (&x)[8])
{
    uint4 u;
    u.x = pack_bf16x2(x[0], x[1]); u.y = pack_bf16x2(x[2], x[3]);
    u.z = pack_bf16x2(x[4], x[5]); u.w = pack_bf16x2(x[6], x[7]);
    *reinterpret_cast<uint4 *>(p) = u;
}

__device__ __forceinline__ void store8(float *p, const float (&x)[8])
{
    reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

// Non-temporal stores, for outputs no later pass of the step reads.
__device__ __forceinline__ void store8_stream(uint16_t *p, const float (&x)[8])
{
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
    __builtin_nontemporal_store(v, reinterpret_cast<v4u *>(p));
}
__device__ __forceinline__ void store8_stream(float *p, const float (&x)[8])
{
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<v4f *>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<v4f *>(p) + 1);
}

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// A piece kept in its storage format until it is summed (fewer registers
// while many rows are in flight).
template <lh_dtype DT> struct Raw8;
template <> struct Raw8<LH_BF16> { uint4 u; };
template <> struct Raw8<LH_F32> { float4 a, b; };

__device__ __forceinline__ void ld_raw(const uint16_t *p, Raw8<LH_BF16> &r) { r.u = *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void ld_raw(const float *p, Raw8<LH_F32> &r)
{
    r.a = reinterpret_cast<const float4 *>(p)[0];
    r.b = reinterpret_cast<const float4 *>(p)[1];
}
// The same for data no later pass reads again (the upstream gradient): a
// non-temporal load, which does not keep the lines in the caches. (The
// inputs Q, K, V are read again by the gather after the front pass, which
// finds part of them still cached: the front pass reads them normally.)
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void ld_stream(const uint16_t *p, Raw8<LH_BF16> &r)
{
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
    r.u = make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void ld_stream(const float *p, Raw8<LH_F32> &r)
{
    const f32x4_nt a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt *>(p));
    const f32x4_nt b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt *>(p) + 1);
    r.a = make_float4(a.x, a.y, a.z, a.w);
    r.b = make_float4(b.x, b.y, b.z, b.w);
}
__device__ __forceinline__ void zero_raw(Raw8<LH_BF16> &r) { r.u = make_uint4(0u, 0u, 0u, 0u); }
__device__ __forceinline__ void zero_raw(Raw8<LH_F32> &r)
{
    r.a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    r.b = r.a;
}
__device__ __forceinline__ void unraw(const Raw8<LH_BF16> &r, float (&x)[8])
{
    const uint4 u = r.u;
    x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xffff0000u);
    x[4] = __uint_as_float(u.z << 16); x[5] = __uint_as_float(u.z & 0xffff0000u);
    x[6] = __uint_as_float(u.w << 16); x[7] = __uint_as_float(u.w & 0xffff0000u);
}
__device__ __forceinline__ void unraw(const Raw8<LH_F32> &r, float (&x)[8])
{
    x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
    x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}

// Workgroup barrier without a memory fence: this wave's LDS accesses are
// complete; its global loads and stores in flight are not waited for.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Element type tags for the layer's inputs / outputs.
// Row kappa(r) of a 32-row block that MFMA operand row r reads: swaps bits 2
// and 3 of r (an involution). With it, register v of lane group g of a
// 32x32 MFMA result holds row 16*(v/8) + 8*g + v%8: runs of 8 consecutive rows.
__device__ __forceinline__ int kappa(int r)
{
    return 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}

// ---------------------------------------------------------------- fp8 lo products
// The second product of an fp16 pair q = hi + lo (q_lo . k) only corrects the
// first, so it runs as a block-scaled fp8 (OCP e4m3) MFMA: x is stored as
// fp8(x * 2^-e) with one exponent e per head and tensor (scale byte 127 + e),
// the smallest that keeps the head's largest magnitude within e4m3's 448.
// Rows far below that maximum lose bits of their lo part, but their logits
// are small by the same factor, so the absolute logit error stays bounded by
// about 2^-15 of the head's largest |q_lo| |k|.
__device__ __forceinline__ int fp8_scale_exp(float amax)
{
    if (!(amax > 0.0f))
        return -127;
    int e = (int)ceilf(__log2f(amax * (1.0f / 448.0f)));
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    while (e < 127 && ldexpf(amax, -e) > 448.0f) // (in case log2 rounded down)
        ++e;
    return e;
}

// 8 values times mul to 8 e4m3 bytes (round to nearest even).
__device__ __forceinline__ uint2 pack8_fp8(const float (&x)[8], float mul)
{
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] * mul, x[1] * mul, 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] * mul, x[3] * mul, w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] * mul, x[5] * mul, 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] * mul, x[7] * mul, w1, true);
    return make_uint2((uint32_t)w0, (uint32_t)w1);
}

// Byte offset, inside a 32-row fp8 tile, of elements 8c .. 8c+7 of row rr.
// The tile is stored in the operand order of v_mfma_scale_f32_32x32x64_f8f6f4:
// fragment m (elements 64m .. 64m+63) is 64 lanes x 32 bytes, lane l holding
// row kappa(l % 32) with byte 8p + j = element 64m + 16p + 8(l/32) + j; each
// fragment is split into two 1 KiB halves (bytes 0-15, then 16-31 of every
// lane) so that a half is one linear 16-byte-per-lane LDS read.
__device__ __forceinline__ int fp8_tile_offset(int rr, int c)
{
    const int m = c >> 3, p = (c & 7) >> 1, h = c & 1;
    return m * 2048 + (p >> 1) * 1024 + (kappa(rr) + 32 * h) * 16 + (p & 1) * 8;
}

template <lh_dtype DT> struct Elem;
template <> struct Elem<LH_BF16> { typedef uint16_t T; };
template <> struct Elem<LH_F32> { typedef float T; };

} // namespace lh
