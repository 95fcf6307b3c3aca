// la_device.h -- device helpers shared by the libla kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// bf16 values are stored as raw 16-bit patterns.
using bf16_t = uint16_t;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> one dword of two bf16 (one v_cvt_pk_bf16_f32, nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Scalar load/store of an element given a runtime dtype (0 = fp32, 1 = bf16).
__device__ __forceinline__ float load_elem(const void *base, int64_t i, int dtype)
{
    return dtype ? bf16_to_f32(static_cast<const uint16_t *>(base)[i])
                 : static_cast<const float *>(base)[i];
}
__device__ __forceinline__ void store_elem(void *base, int64_t i, int dtype, float v)
{
    if (dtype) static_cast<uint16_t *>(base)[i] = f32_to_bf16(v);
    else static_cast<float *>(base)[i] = v;
}

// Scalar load/store with the dtype as a template parameter (float or bf16_t).
template <typename T> __device__ __forceinline__ float ld(const void *base, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const void *base, int64_t i)
{
    return static_cast<const float *>(base)[i];
}
template <> __device__ __forceinline__ float ld<bf16_t>(const void *base, int64_t i)
{
    return bf16_to_f32(static_cast<const uint16_t *>(base)[i]);
}
template <typename T> __device__ __forceinline__ void st(void *base, int64_t i, float v);
template <> __device__ __forceinline__ void st<float>(void *base, int64_t i, float v)
{
    static_cast<float *>(base)[i] = v;
}
template <> __device__ __forceinline__ void st<bf16_t>(void *base, int64_t i, float v)
{
    static_cast<uint16_t *>(base)[i] = f32_to_bf16(v);
}

// Element storage traits for the templated state dtype.
template <typename T> struct Stor;
template <> struct Stor<float> {
    static constexpr int kPer16B = 4;
    __device__ static __forceinline__ void unpack(const uint4 &r, float *f)
    {
        f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
    }
    __device__ static __forceinline__ uint4 pack(const float *f)
    {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                          __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
};
template <> struct Stor<bf16_t> {
    static constexpr int kPer16B = 8;
    __device__ static __forceinline__ void unpack(const uint4 &r, float *f)
    {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
        f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
    }
    __device__ static __forceinline__ uint4 pack(const float *f)
    {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                          pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
};

// Cross-lane moves.  DPP controls: quad_perm [1,0,3,2] = 0xB1,
// quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
// bound_ctrl is set so the move folds into the consuming add (v_add_f32_dpp);
// every pattern used here reads in-range lanes only.
// 16-byte streaming load / store with the non-temporal hint: state rows are
// touched once per call, so they should not displace reusable lines in the
// caches.  Measured on the decode kernel, hinting both directions shortens a
// 55 MB launch by about a sixth.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void *p)
{
    const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void *p, uint4 v)
{
    const u32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, static_cast<u32x4_t *>(p));
}

template <int CTRL> __device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Exchange with lane ^ 16 inside each 32-lane half (ds_swizzle bitmask mode:
// and 0x1F, or 0, xor 0x10).
__device__ __forceinline__ float swz_xor16(float x)
{
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

// Sum over aligned groups of N consecutive lanes (N = 1, 2, 4, 8, 16, 32);
// every lane of a group receives the bitwise-identical total (each step adds
// a commuted pair, so all lanes see the same operands).
template <int N> __device__ __forceinline__ float group_sum(float x)
{
    if constexpr (N >= 2) x += dpp_mov<0xB1>(x);
    if constexpr (N >= 4) x += dpp_mov<0x4E>(x);
    if constexpr (N >= 8) x += dpp_mov<0x141>(x);
    if constexpr (N >= 16) x += dpp_mov<0x140>(x);
    if constexpr (N >= 32) x += swz_xor16(x);
    return x;
}

// Sum over the whole wave; the result is wave-uniform.
__device__ __forceinline__ float wave_sum(float x)
{
    x = group_sum<32>(x);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
}

// exp via the hardware exp2 (v_exp_f32) of the fp32 product x log2(e): the
// rounding of that product (and of log2(e) itself) adds a relative error of
// up to about 1.25 |x| 2^-24, so the error grows with |x| (a few ulp for the
// modest log-decays and conv activations it serves; bounded in
// tests/test_gpu_device_math.py).
__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// exp(x) accurate to about 2 ulp over the whole fp32 range, for the chunked
// prefill, whose differences of running log-decay sums reach |x| of
// hundreds.  t = x log2(e) is carried as an unevaluated sum t_hi + t_lo:
// t_hi = fl(x c_hi) and its exact rounding error from one FMA (the
// error-free product of Ogita, Rump and Oishi, "Accurate sum and dot
// product", SIAM J. Sci. Comput. 26, 2005), plus x c_lo for the part of
// log2(e) beyond fp32 (c_hi + c_lo = log2(e) to about 2^-50).  Then
// 2^t = 2^t_hi 2^t_lo with 2^t_lo = 1 + t_lo ln 2 to second order, since
// |t_lo| <= ulp(t_hi).  Bounded against fp64 exp in
// tests/test_gpu_device_math.py.
__device__ __forceinline__ float exp_acc(float x)
{
    const float kHi = 1.44269502162933349609375f, kLo = 1.925963033500011e-8f;
    const float t = x * kHi;
    float e = fmaf(x, kHi, -t);
    e = fmaf(x, kLo, e);
    return __builtin_amdgcn_exp2f(t) * fmaf(e, 0.69314718f, 1.0f);
}
__device__ __forceinline__ float silu(float y)
{
    return y * __builtin_amdgcn_rcpf(1.0f + fast_exp(-y));
}

}  // namespace la
