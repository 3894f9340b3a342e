// moe_device.h -- device helpers shared by the MoE decode kernels (gfx950): format conversions,
// MX block dot products, lane exchanges and reductions, top-k keys.  Private to the library.
#pragma once
#ifndef __HIPCC_RTC__
#include <hip/hip_runtime.h>
#include <stdint.h>
#else  // hipRTC provides the runtime header itself, and the fixed-width integer types in a namespace
using __hip_internal::int32_t;
using __hip_internal::int64_t;
using __hip_internal::uint16_t;
using __hip_internal::uint32_t;
using __hip_internal::uint64_t;
using __hip_internal::uint8_t;
#endif

namespace moe {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------------------------------
// small helpers
// ------------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float((b & 0xffffu) << 16); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// E8M0 byte -> fp32 2^(b-127) (OCP MX): b in the fp32 exponent field for 1 <= b <= 254; b = 0 is
// 2^-127, the fp32 subnormal 0x00400000; b = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    b &= 0xffu;
    const uint32_t u = b == 0u ? 0x00400000u : b == 255u ? 0x7fc00000u : b << 23;
    return __uint_as_float(u);
}

// E4M3 NaN code with the sign of the fp32 NaN v: S.1111.111 (the hardware conversion writes 0xFF
// for every NaN).
__device__ __forceinline__ uint32_t e4m3_nan(float v) { return ((__float_as_uint(v) >> 24) & 0x80u) | 0x7fu; }

// Two fp32 values -> two OCP E4M3 codes (round to nearest even, saturating to +-448) in the low 16
// bits; a NaN keeps its sign.
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b) {
    uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
    if (__builtin_isnan(a)) c = (c & 0xff00u) | e4m3_nan(a);
    if (__builtin_isnan(b)) c = (c & 0x00ffu) | (e4m3_nan(b) << 8);
    return c;
}

// Two E4M3 codes (low 16 bits) -> their exact f16 values.
__device__ __forceinline__ half2_t e4m3x2_to_f16x2(uint32_t packed) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)packed, 1.0f, false);
}

// Byte B of a dword (two E2M1 codes, even element in the low nibble) -> two f16 values.
template <int B>
__device__ __forceinline__ half2_t e2m1x2_to_f16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B);
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ __forceinline__ uint32_t comp(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Streaming (non-temporal) loads of weights that are read once per pass.
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt(const uint2* p) {
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
    return make_uint2(v.x, v.y);
}

// Dot product of one 16-byte MX block (32 E2M1 codes) with 32 f16 activations per token (xp[j]
// points at the block's 16 half2 pairs in LDS), accumulated into p in fp32.  Every product is
// exact in fp32.  Activations are read per dword of codes to keep few registers live.
template <int NT>
__device__ __forceinline__ void block_dot(const uint4& w, const half2_t* const (&xp)[NT], float (&p)[NT], int nt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t wd = comp(w, q);
        const half2_t w0 = e2m1x2_to_f16x2<0>(wd);
        const half2_t w1 = e2m1x2_to_f16x2<1>(wd);
        const half2_t w2 = e2m1x2_to_f16x2<2>(wd);
        const half2_t w3 = e2m1x2_to_f16x2<3>(wd);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (j < nt) {
                const uint4 x = *(const uint4*)(xp[j] + 4 * q);
                p[j] = __builtin_amdgcn_fdot2(w0, as_h2(x.x), p[j], false);
                p[j] = __builtin_amdgcn_fdot2(w1, as_h2(x.y), p[j], false);
                p[j] = __builtin_amdgcn_fdot2(w2, as_h2(x.z), p[j], false);
                p[j] = __builtin_amdgcn_fdot2(w3, as_h2(x.w), p[j], false);
            }
        }
    }
}

// The same for nt tokens of at most NT: a work item with one token (every shared-expert item, and
// every routed expert when the tokens' top-k sets are disjoint) takes the one-token form, without
// the per-token guards that the NT form carries through each dword.
template <int NT>
__device__ __forceinline__ void block_dot_nt(const uint4& w, const half2_t* const (&xp)[NT], float (&p)[NT], int nt) {
    if constexpr (NT > 1) {
        if (nt == 1) {
            const half2_t* const x1[1] = {xp[0]};
            float p1[1] = {p[0]};
            block_dot<1>(w, x1, p1, 1);
            p[0] = p1[0];
            return;
        }
    }
    block_dot<NT>(w, xp, p, nt);
}

// Lane exchange without LDS: stage S pairs every lane with one partner (0: lane^1, 1: lane^2,
// 2: mirror within 8 lanes, 3: mirror within 16 lanes, 4: lane^16, 5: lane^32).  Applying an
// associative, commutative op with stages 0..n-1 reduces over groups of 2^n lanes.
template <int S>
__device__ __forceinline__ uint32_t xchg(uint32_t v) {
    if constexpr (S == 0) return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, true);   // quad_perm 1,0,3,2
    else if constexpr (S == 1) return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, true);  // quad_perm 2,3,0,1
    else if constexpr (S == 2) return __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, true);  // row_half_mirror
    else if constexpr (S == 3) return __builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, true);  // row_mirror
    else if constexpr (S == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return ((threadIdx.x >> 5) & 1) ? r[0] : r[1];
    }
}
template <int S>
__device__ __forceinline__ float xchg(float v) { return __uint_as_float(xchg<S>(__float_as_uint(v))); }
template <int S>
__device__ __forceinline__ double xchg(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t r = ((uint64_t)xchg<S>((uint32_t)(u >> 32)) << 32) | xchg<S>((uint32_t)u);
    return __builtin_bit_cast(double, r);
}
template <int S>
__device__ __forceinline__ uint64_t xchg(uint64_t u) {
    return ((uint64_t)xchg<S>((uint32_t)(u >> 32)) << 32) | xchg<S>((uint32_t)u);
}

// max over groups of 16 lanes / over the wave; sums over the wave (every lane gets the result)
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, xchg<0>(v));
    v = fmaxf(v, xchg<1>(v));
    v = fmaxf(v, xchg<2>(v));
    return fmaxf(v, xchg<3>(v));
}
__device__ __forceinline__ float max64(float v) {
    v = max16(v);
    v = fmaxf(v, xchg<4>(v));
    return fmaxf(v, xchg<5>(v));
}
__device__ __forceinline__ float sum64(float v) {
    v += xchg<0>(v);
    v += xchg<1>(v);
    v += xchg<2>(v);
    v += xchg<3>(v);
    v += xchg<4>(v);
    return v + xchg<5>(v);
}
__device__ __forceinline__ double sum64(double v) {
    v += xchg<0>(v);
    v += xchg<1>(v);
    v += xchg<2>(v);
    v += xchg<3>(v);
    v += xchg<4>(v);
    return v + xchg<5>(v);
}
// sum over the KSUB consecutive lanes of a row group (KSUB = 1, 2, 4 or 8)
template <int KSUB>
__device__ __forceinline__ float sum_ksub(float v) {
    if constexpr (KSUB >= 2) v += xchg<0>(v);
    if constexpr (KSUB >= 4) v += xchg<1>(v);
    if constexpr (KSUB >= 8) v += xchg<2>(v);
    return v;
}

// Order-preserving 64-bit key of (logit, expert): larger logit first, then lower index first.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
    const uint32_t u = __float_as_uint(v + 0.0f);  // -0 -> +0
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t max64u(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ void cx_desc(uint64_t& a, uint64_t& b) {
    const uint64_t hi = max64u(a, b), lo = a > b ? b : a;
    a = hi;
    b = lo;
}

}  // namespace moe
