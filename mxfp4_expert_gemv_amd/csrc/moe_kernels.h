// moe_kernels.h -- device code of the W4A8 sparse-MoE decode kernels (gfx950): the kernels, their
// argument structs and the pieces they share.  Compiled ahead of time into the library (through
// moe_kernels.hip) and, for one layer shape at a time, at run time by hipRTC (moe_jit.cpp): there
// the macros MOE_SHAPE_H, _E, _K, _S, _I and _NORM fix the layer's shape and input normalisation at
// compile time (MOE_SHAPE below), so that the compiler folds the divisions and loop bounds that the
// shape-generic ahead-of-time build takes from the kernel arguments; moe_kernels_flash.hip does the
// same ahead of time for one shape (each macro left undefined stays a run-time value).  Private to
// the library.
#pragma once
#include "moe_device.h"
#include "moe_layout.h"

// MOE_SHAPE(name, runtime): the compile-time constant MOE_SHAPE_<name> where the build defines it,
// else the run-time expression.
#define MOE_SHAPE(name, runtime) MOE_SHAPE_SEL_##name(runtime)
#ifdef MOE_SHAPE_H
#define MOE_SHAPE_SEL_H(r) (MOE_SHAPE_H)
#else
#define MOE_SHAPE_SEL_H(r) (r)
#endif
#ifdef MOE_SHAPE_E
#define MOE_SHAPE_SEL_E(r) (MOE_SHAPE_E)
#else
#define MOE_SHAPE_SEL_E(r) (r)
#endif
#ifdef MOE_SHAPE_K
#define MOE_SHAPE_SEL_K(r) (MOE_SHAPE_K)
#else
#define MOE_SHAPE_SEL_K(r) (r)
#endif
#ifdef MOE_SHAPE_S
#define MOE_SHAPE_SEL_S(r) (MOE_SHAPE_S)
#else
#define MOE_SHAPE_SEL_S(r) (r)
#endif
#ifdef MOE_SHAPE_I
#define MOE_SHAPE_SEL_I(r) (MOE_SHAPE_I)
#else
#define MOE_SHAPE_SEL_I(r) (r)
#endif
#ifdef MOE_SHAPE_NORM
#define MOE_SHAPE_SEL_NORM(r) (MOE_SHAPE_NORM)
#else
#define MOE_SHAPE_SEL_NORM(r) (r)
#endif

// Namespace of the kernels and their argument structs: moe, or a nested one in a build with the
// shape folded in ahead of time (moe_kernels_flash.hip), so that both builds link into one library.
#ifndef MOE_KERNELS_NS_BEGIN
#define MOE_KERNELS_NS_BEGIN namespace moe {
#define MOE_KERNELS_NS_END }
#endif

MOE_KERNELS_NS_BEGIN

// Timing record of a graph-replayed pass (moe_decode_timing_enable, mode 1): the kernels' STAMP
// instances write, from thread 0 of every workgroup, the device's constant-rate wall clock at the
// workgroup's start (stamp[2 b]) and, after a final barrier, at its end (stamp[2 b + 1]).  The other
// instances, those of normal runs, carry none of this.
template <bool STAMP>
__device__ __forceinline__ void stamp_start(unsigned long long* s) {
    if constexpr (STAMP)
        if (threadIdx.x == 0) s[2 * blockIdx.x] = __builtin_amdgcn_s_memrealtime();
}
template <bool STAMP>
__device__ __forceinline__ void stamp_end(unsigned long long* s) {
    if constexpr (STAMP) {
        __syncthreads();
        if (threadIdx.x == 0) s[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
    }
}


// Scale bytes of one lane: BPL = 8 -> 8 bytes, BPL = 4 -> 4 bytes.
template <int BPL>
struct ScaleBytes;
template <>
struct ScaleBytes<8> {
    uint2 v;
    __device__ void load(const uint8_t* p) { v = ld_nt((const uint2*)p); }
    __device__ uint32_t get(int i) const { return (i < 4 ? v.x >> (8 * i) : v.y >> (8 * (i - 4))) & 0xffu; }
};
template <>
struct ScaleBytes<4> {
    uint32_t v;
    __device__ void load(const uint8_t* p) { v = __builtin_nontemporal_load((const uint32_t*)p); }
    __device__ uint32_t get(int i) const { return (v >> (8 * i)) & 0xffu; }
};

// ------------------------------------------------------------------------------------------------
// shared pieces: MoE input, FP8 quantisation of the input, gate/up tile
// ------------------------------------------------------------------------------------------------

// The MoE input of T tokens in one workgroup, in two steps so that the caller can issue the load of
// x before other loads (the loads of a wave complete in issue order):
// moe_input_load: this thread's 8-element chunk of every token of x (threads past H / 8 load none).
// moe_input_finish: x_in = x, or bf16(fl32(x * r)) with r = 1 / sqrt(mean(x^2) + 1e-6) evaluated in
// fp64 (sum of squares in fp64), staged in LDS xb[T][H]; and its per-token FP8 scale
// s = max|x_in| / 448 (1 when x_in = 0), returned in sx.  The maximum of |x_in| is bf16(max|x| * r)
// because rounding is monotonic, so both reductions share one barrier.  red_d, red_m: LDS
// [waves][T].  Ends with a barrier.
template <int T>
__device__ __forceinline__ void moe_input_load(const uint16_t* __restrict__ x, int H, uint4 (&v)[T]) {
    const int tid = threadIdx.x, NC = H / 8;
#pragma unroll
    for (int t = 0; t < T; ++t)
        if (tid < NC) v[t] = *(const uint4*)(x + (size_t)t * H + tid * 8);
}

template <int T>
__device__ void moe_input_finish(uint4 (&v)[T], int H, bool normalize, uint16_t* xb, double* red_d, float* red_m,
                                 float (&sx)[T]) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, NW = blockDim.x >> 6, NC = H / 8;
    const bool has = tid < NC;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        float m = 0.0f;
        if (has) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float a = bf16_to_f32(comp(v[t], q)), b = bf16_to_f32(comp(v[t], q) >> 16);
                ss += (double)a * (double)a + (double)b * (double)b;
                m = fmaxf(m, fmaxf(fabsf(a), fabsf(b)));
            }
        }
        if (normalize) ss = sum64(ss);
        m = max64(m);
        if (lane == 0) {
            red_d[wv * T + t] = ss;
            red_m[wv * T + t] = m;
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        float m = 0.0f;
        for (int w = 0; w < NW; ++w) {
            ss += red_d[w * T + t];
            m = fmaxf(m, red_m[w * T + t]);
        }
        if (normalize) {
            const double r = 1.0 / sqrt(ss / (double)H + 1e-6);
            m = bf16_to_f32(f32_to_bf16((float)((double)m * r)));
            if (has) {
                uint32_t o[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t d = comp(v[t], q);
                    const uint32_t lo = f32_to_bf16((float)((double)bf16_to_f32(d) * r));
                    const uint32_t hi = f32_to_bf16((float)((double)bf16_to_f32(d >> 16) * r));
                    o[q] = lo | (hi << 16);
                }
                v[t] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
        sx[t] = m > 0.0f ? m / 448.0f : 1.0f;
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
        if (has) *(uint4*)(xb + t * H + tid * 8) = v[t];
    __syncthreads();
}

// FP8 codes RNE(x_in / s) of this workgroup's share of the 8-element units of xb[T][H] (LDS,
// complete): every workgroup of the grid stores its own share (workgroup 0 also the scales), so
// the work on each workgroup's path is one division per element of its share.  codes_dbg /
// scale_dbg: optional copies.
template <int T>
__device__ void quantize_slice(const uint16_t* xb, int H, const float (&sx)[T], uint8_t* codes, float* scales,
                               uint8_t* codes_dbg, float* scale_dbg) {
    const int tid = threadIdx.x, NC = H / 8;
    const int per = (NC + (int)gridDim.x - 1) / (int)gridDim.x, u = (int)blockIdx.x * per + tid;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if (blockIdx.x == 0 && tid == 0) {
            scales[t] = sx[t];
            if (scale_dbg) scale_dbg[t] = sx[t];
        }
        if (tid < per && u < NC) {
            const uint4 v = *(const uint4*)(xb + t * H + u * 8);
            uint32_t c[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t d = comp(v, q);
                c[q] = e4m3_pack2(bf16_to_f32(d) / sx[t], bf16_to_f32(d >> 16) / sx[t]);
            }
            const uint2 cw = make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
            *(uint2*)(codes + (size_t)t * H + u * 8) = cw;
            if (codes_dbg) *(uint2*)(codes_dbg + (size_t)t * H + u * 8) = cw;
        }
    }
}

// The MoE input of T tokens, computed by one workgroup: x_in = x, or bf16(fl32(x * r)) with
// r = 1 / sqrt(mean(x^2) + 1e-6) evaluated in fp64 (sum of squares in fp64); its per-token FP8
// quantisation s = max|x_in| / 448 (1 when x_in = 0), codes = RNE(x_in / s).  The maximum of
// |x_in| is bf16(max|x| * r) because rounding is monotonic.  x is staged in LDS xb[T][H].  Writes
// x_in (bf16) to xn, the codes to xq, the scales to xs, and the optional per-layer copies (trace:
// x itself; x_scale; x_codes).
template <int T>
__device__ void norm_quant(const uint16_t* x, int H, bool normalize, uint16_t* xb, uint16_t* xn, uint8_t* xq,
                           float* xs, uint16_t* trace, float* x_scale, uint8_t* x_codes, double* redd, float* redf) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, NW = blockDim.x >> 6, nth = blockDim.x;
    const int NQ = H / 4;  // 4-element quads per token
    double ss[T];
    float mx[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        ss[t] = 0.0;
        mx[t] = 0.0f;
    }
    for (int i = tid; i < T * NQ; i += nth) {
        int t = 0;
#pragma unroll
        for (int tt = 1; tt < T; ++tt) t += i >= tt * NQ ? 1 : 0;
        const uint64_t v = ((const uint64_t*)x)[i];
        ((uint64_t*)xb)[i] = v;
        if (trace) ((uint64_t*)trace)[i] = v;
        double d = 0.0;
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float xv = bf16_to_f32((uint32_t)(v >> (16 * q)));
            m = fmaxf(m, fabsf(xv));
            d = fma((double)xv, (double)xv, d);
        }
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
            if (tt == t) {
                ss[tt] += d;
                mx[tt] = fmaxf(mx[tt], m);
            }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const double sv = normalize ? sum64(ss[t]) : 0.0;
        const float mv = max64(mx[t]);
        if (lane == 0) {
            redd[wv * T + t] = sv;
            redf[wv * T + t] = mv;
        }
    }
    __syncthreads();
    double rr[T];
    float sxv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        double sv = 0.0;
        float mv = 0.0f;
        for (int q = 0; q < NW; ++q) {
            sv += redd[q * T + t];
            mv = fmaxf(mv, redf[q * T + t]);
        }
        double r = 1.0;
        if (normalize) {
            r = 1.0 / sqrt(sv / (double)H + 1e-6);
            mv = bf16_to_f32(f32_to_bf16((float)((double)mv * r)));
        }
        rr[t] = r;
        sxv[t] = mv > 0.0f ? mv / 448.0f : 1.0f;
    }
    if (tid < T) {
        float sv = sxv[0];
#pragma unroll
        for (int t = 1; t < T; ++t)
            if (tid == t) sv = sxv[t];
        xs[tid] = sv;
        if (x_scale) x_scale[tid] = sv;
    }
    for (int i = tid; i < T * NQ; i += nth) {
        int t = 0;
#pragma unroll
        for (int tt = 1; tt < T; ++tt) t += i >= tt * NQ ? 1 : 0;
        double r = rr[0];
        float sv = sxv[0];
#pragma unroll
        for (int tt = 1; tt < T; ++tt)
            if (t == tt) {
                r = rr[tt];
                sv = sxv[tt];
            }
        uint2 v = ((const uint2*)xb)[i];
        if (normalize) {
            uint32_t o[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const uint32_t d = q ? v.y : v.x;
                const uint32_t lo = f32_to_bf16((float)((double)bf16_to_f32(d) * r));
                const uint32_t hi = f32_to_bf16((float)((double)bf16_to_f32(d >> 16) * r));
                o[q] = lo | (hi << 16);
            }
            v = make_uint2(o[0], o[1]);
        }
        ((uint2*)xn)[i] = v;
        const uint32_t c0 = e4m3_pack2(bf16_to_f32(v.x) / sv, bf16_to_f32(v.x >> 16) / sv);
        const uint32_t c1 = e4m3_pack2(bf16_to_f32(v.y) / sv, bf16_to_f32(v.y >> 16) / sv);
        ((uint32_t*)xq)[i] = c0 | (c1 << 16);
        if (x_codes) ((uint32_t*)x_codes)[i] = c0 | (c1 << 16);
    }
}

template <int BPL>
struct GuLoads {
    uint4 w[BPL];
    ScaleBytes<BPL> s;
    uint4 sm[BPL / 4];  // MF: the scale bytes of the lane's gate row, then of its up row (4 BPL)
    // expert e, tile `tile` of `tiles`, this wave's BPL steps; MF: the matrix-core layout, whose
    // scale bytes are shared by the four lanes of a row (one address, one fetch)
    template <bool MF = false>
    __device__ void issue(const uint4* w13, const uint8_t* w13s, int e, int tile, int tiles, int GW) {
        const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
        const size_t base = (((size_t)e * tiles + tile) * GW + wv);
        const uint4* p = w13 + base * BPL * kWave + lane;
#pragma unroll
        for (int i = 0; i < BPL; ++i) w[i] = ld_nt(p + i * kWave);
        if constexpr (MF) {
            const uint4* q = (const uint4*)(w13s + (base * 16 + (lane & 15)) * (4 * BPL));
#pragma unroll
            for (int i = 0; i < BPL / 4; ++i) sm[i] = ld_nt(q + i);
        } else {
            s.load(w13s + (base * kWave + lane) * BPL);
        }
    }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 8 E2M1 codes (a dword, even element in the low nibble of each byte) times the block scale ->
// the bf16 A operand of one MFMA block.  v_cvt_scalef32_pk_bf16_fp4 takes the scale as the
// exponent field of an f32 operand, read as E8M0 (mantissa and sign ignored: 0 is 2^-127, 255 is
// NaN), so the operand is the scale byte shifted into that field.  The result is code x scale
// exactly for every E8M0 byte: bf16 has the fp32 exponent range (0.5 x 2^-127 is a bf16
// subnormal, 6 x 2^127 overflows to inf as in fp32; measured for all 16 codes).
__device__ __forceinline__ bf16x8_t e2m1x8_to_bf16x8(uint32_t d, uint32_t scale_byte) {
    const float scale = __uint_as_float(scale_byte << 23);
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, scale, 3);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 E4M3 codes (two dwords) -> 8 bf16 (exact).
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 c) {
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, true)));
}

template <int BPL>
__device__ __forceinline__ uint32_t scale_byte(const GuLoads<BPL>& L, int k) {
    const uint4& v = L.sm[k >> 4];
    const uint32_t d = (k & 15) < 4 ? v.x : (k & 15) < 8 ? v.y : (k & 15) < 12 ? v.z : v.w;
    return (d >> (8 * (k & 3))) & 0xffu;
}

// Matrix-core form of the gate/up dot products (weights repacked for it, MOE_F_MFMA): each of the
// wave's 2 BPL MX blocks is one v_mfma_f32_16x16x32_bf16 for the 16 gate rows and one for the 16
// up rows of the tile.  A: lane l holds row l % 16 and K 8 (l / 16) .. +8 of the block (a dword of
// its units: gate units 0 .. BPL/2-1, up units after them, four blocks per unit), converted with
// the block scale; B: column n = l % 16 is the expert's n-th token (zero columns past its tokens),
// the same K from xb (LDS, [T][H] bf16 of the input's E4M3 codes).  The per-token fp32 scale is
// applied afterwards, as in the VALU form.  Measured on gfx950, one such instruction is within
// 2.7 * 2^-24 * sum |terms| of the exact C + 32 products: the accuracy of fp32 accumulation.  The
// tile's partial sums go to red in the VALU form's layout.
template <int T, int BPL>
__device__ void gateup_dot_mfma(const GuLoads<BPL>& L, const uint16_t* xb, int H, int nt, const int (&tok)[T],
                                float* red) {
    constexpr int BW = 2 * BPL;  // MX blocks per wave
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
    int tk = 0;
#pragma unroll
    for (int j = 0; j < T; ++j)
        if (n == j) tk = tok[j];
    const bool on = n < nt;
    const uint16_t* xr = xb + (size_t)tk * H + wv * BW * kBlock + 8 * g;
    // one accumulator per matrix: two (shorter chains) took 76 VGPRs, one wave less per SIMD, and
    // measured slower; capping registers at 64 spilled
    f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < BW; ++j) {
        uint4 xv = make_uint4(0, 0, 0, 0);
        if (on) xv = *(const uint4*)(xr + j * kBlock);
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xv);
        const uint4& wg = L.w[j >> 2];
        const uint4& wu = L.w[BPL / 2 + (j >> 2)];
        const uint32_t dg = (j & 3) == 0 ? wg.x : (j & 3) == 1 ? wg.y : (j & 3) == 2 ? wg.z : wg.w;
        const uint32_t du = (j & 3) == 0 ? wu.x : (j & 3) == 1 ? wu.y : (j & 3) == 2 ? wu.z : wu.w;
        const bf16x8_t ag = e2m1x8_to_bf16x8(dg, scale_byte(L, j));
        const bf16x8_t au = e2m1x8_to_bf16x8(du, scale_byte(L, BW + j));
        accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, b, accg, 0, 0, 0);
        accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au, b, accu, 0, 0, 0);
    }
    if (on) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            red[(wv * T + n) * kGuRows + 4 * g + i] = accg[i];
            red[(wv * T + n) * kGuRows + kGuOut + 4 * g + i] = accu[i];
        }
    }
}

// LDS fill of the input's 8 E4M3 codes of thread slot i (bytes 8 i .. 8 i + 7 of token t's row):
// f16 pairs [T][H/2] for the VALU form, bf16 [T][H] for the matrix-core form (MF).
template <bool MF>
__device__ __forceinline__ void store_codes(void* xact, int H, int t, int i, uint2 c) {
    if constexpr (MF) {
        *(uint4*)((uint16_t*)xact + (size_t)t * H + i * 8) = e4m3x8_to_bf16x8(c);
    } else {
        half2_t* o = (half2_t*)xact + t * (H / 2) + i * 4;
        o[0] = e4m3x2_to_f16x2(c.x & 0xffffu);
        o[1] = e4m3x2_to_f16x2(c.x >> 16);
        o[2] = e4m3x2_to_f16x2(c.y & 0xffffu);
        o[3] = e4m3x2_to_f16x2(c.y >> 16);
    }
}

// The gate/up tile of one expert: 16 gate + 16 up rows over all H, for the nt tokens tok[j] (their
// h goes to pair pair[j]); sx: LDS scales per token.  red: LDS [kMaxWaves][T][32].  xact: LDS
// activations, f16 pairs [T][H/2] (VALU form) or bf16 [T][H] (MF, the matrix-core form).
template <int T, int BPL, bool MF = false>
__device__ void gateup_tile(const GuLoads<BPL>& L, const void* xact, int H, const float* sx, int nt,
                            const int (&tok)[T], const int (&pair)[T], int tile, int I, float* h, float* hamax,
                            float* red) {
    const int tid = threadIdx.x, nth = blockDim.x, lane = tid & 63, wv = tid >> 6, NW = nth >> 6, Hh = H / 2;
    if constexpr (MF) {
        gateup_dot_mfma<T, BPL>(L, (const uint16_t*)xact, H, nt, tok, red);
    } else {
    const half2_t* xh = (const half2_t*)xact;
    const int ks = lane & 1;
    float acc[T];
#pragma unroll
    for (int j = 0; j < T; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
        const float scale = e8m0_to_f32(L.s.get(i));
        const int pbase = ((wv * BPL + i) * 2 + ks) * (kBlock / 2);
        const half2_t* xp[T];
#pragma unroll
        for (int j = 0; j < T; ++j) xp[j] = xh + tok[j] * Hh + pbase;
        float p[T];
#pragma unroll
        for (int j = 0; j < T; ++j) p[j] = 0.0f;
        block_dot_nt<T>(L.w[i], xp, p, nt);
#pragma unroll
        for (int j = 0; j < T; ++j) acc[j] = fmaf(p[j], scale, acc[j]);
        __builtin_amdgcn_sched_barrier(0);  // bound the live activation registers to one block
    }
#pragma unroll
    for (int j = 0; j < T; ++j) {
        acc[j] += xchg<0>(acc[j]);
        if (j < nt && ks == 0) red[(wv * T + j) * kGuRows + (lane >> 1)] = acc[j];
    }
    }
    __syncthreads();
    const int tiles = I / kGuOut;
    for (int base = 0; base < kGuOut * nt; base += nth) {
        const int idx = base + tid, j = idx >> 4, r = idx & 15;
        const bool act = idx < kGuOut * nt;
        float hv = 0.0f;
        int pj = 0;
        if (act) {
            float g = 0.0f, u = 0.0f;
            for (int w = 0; w < NW; ++w) {
                g += red[(w * T + j) * kGuRows + r];
                u += red[(w * T + j) * kGuRows + kGuOut + r];
            }
            int tk = tok[0];
            pj = pair[0];
#pragma unroll
            for (int q = 1; q < T; ++q)
                if (j == q) {
                    tk = tok[q];
                    pj = pair[q];
                }
            const float s = sx[tk];
            g *= s;
            u *= s;
            hv = g / (1.0f + expf(-g)) * u;
            h[(size_t)pj * I + tile * kGuOut + r] = hv;
        }
        const float m = max16(fabsf(hv));
        if (act && r == 0) hamax[(size_t)pj * tiles + tile] = m;
    }
}

// Top-k.  One wave takes the top-k of a run of 64 P consecutive experts: lane l holds experts
// base + P l .. base + P l + P - 1 and sorts them by (logit descending, index ascending) with
// 64-bit keys; then each of the k rounds takes the wave-wide maximum of the lanes' head logits
// (32-bit order-preserving codes) through lane exchanges, the lowest lane holding it wins (lower
// lanes hold lower experts, so ties go to the lower index) and pops its head.  Lane r keeps the
// winner of round r.  With one wave per token (P = 8) that is the answer; with W waves per token
// (P = 8 / W) the first wave of the token merges the W candidate lists the same way, one
// candidate per lane in (wave, rank) order, which again sends ties to the lower index.  The
// softmax over the selected logits runs across lanes 0..k-1.  (A six-level bitonic merge tree
// across lanes, and 64-bit keys in the rounds, measured slower: a single wave is bound by its
// instruction count.)  Then the list of distinct routed experts; everything lands in LDS.
//
// route_issue loads the logits so that the caller can overlap other work with their latency;
// route_finish completes the selection (on small workgroups, tokens beyond the waves are loaded
// there).

// P logits of this lane from row[base + P lane ..] (E a multiple of 8; lanes past E reload the
// last P, their keys are dropped).
template <int P>
__device__ __forceinline__ void load_logits(const float* row, int base, int E, float (&v)[P]) {
    const float* p = row + min(base + (int)(threadIdx.x & 63) * P, E - P);
    if constexpr (P == 8) {
        const float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else if constexpr (P == 4) {
        const float4 a = *(const float4*)p;
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    } else {
        const float2 a = *(const float2*)p;
        v[0] = a.x; v[1] = a.y;
    }
}

// The same from logits that other workgroups of the running kernel stored with device-scope stores
// (64-bit device-scope loads: the logits are 8-byte aligned).
__device__ __forceinline__ void load_logits8_agent(const float* row, int E, float (&v)[8]) {
    const uint64_t* p = (const uint64_t*)(row + min((int)(threadIdx.x & 63) * 8, E - 8));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint64_t u = __hip_atomic_load(p + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v[2 * j] = __uint_as_float((uint32_t)u);
        v[2 * j + 1] = __uint_as_float((uint32_t)(u >> 32));
    }
}

// W waves per token: wave v takes token v / W, experts (v % W) 64 P ...  Every wave loads (waves
// past the last token repeat it), so that the number of loads in flight is the same on every path
// and later waits stay exact.
template <int T, int W>
__device__ __forceinline__ void route_issue(const float* logits, int E, float (&lgv)[8 / W]) {
    constexpr int P = 8 / W;
    const int wv = threadIdx.x >> 6, t = min(wv / W, T - 1);
    load_logits<P>(logits + t * E, (wv % W) * 64 * P, E, lgv);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
    m = max(m, xchg<0>(m));
    m = max(m, xchg<1>(m));
    m = max(m, xchg<2>(m));
    m = max(m, xchg<3>(m));
    m = max(m, xchg<4>(m));
    return max(m, xchg<5>(m));
}

// One wave's top-k of its P logits per lane (experts base + P lane + j): lane r < k returns the
// order code and expert of rank r.
template <int P>
__device__ __forceinline__ void wave_topk(const float (&lgv)[P], int base, int E, int k, uint32_t& my_code,
                                          int& my_id) {
    const int lane = threadIdx.x & 63;
    uint64_t key[P];  // order code of the logit above, 7 - j below; 0 = no expert
#pragma unroll
    for (int j = 0; j < P; ++j) {
        const uint32_t u = __float_as_uint(lgv[j] + 0.0f);  // -0 -> +0
        const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        key[j] = base + lane * P + j < E ? ((uint64_t)o << 32) | (uint32_t)(7 - j) : 0ull;
    }
    if constexpr (P == 8) {
        cx_desc(key[0], key[1]); cx_desc(key[2], key[3]); cx_desc(key[4], key[5]); cx_desc(key[6], key[7]);
        cx_desc(key[0], key[2]); cx_desc(key[1], key[3]); cx_desc(key[4], key[6]); cx_desc(key[5], key[7]);
        cx_desc(key[1], key[2]); cx_desc(key[5], key[6]);
        cx_desc(key[0], key[4]); cx_desc(key[1], key[5]); cx_desc(key[2], key[6]); cx_desc(key[3], key[7]);
        cx_desc(key[2], key[4]); cx_desc(key[3], key[5]);
        cx_desc(key[1], key[2]); cx_desc(key[3], key[4]); cx_desc(key[5], key[6]);
    } else if constexpr (P == 4) {
        cx_desc(key[0], key[1]); cx_desc(key[2], key[3]);
        cx_desc(key[0], key[2]); cx_desc(key[1], key[3]);
        cx_desc(key[1], key[2]);
    } else {
        cx_desc(key[0], key[1]);
    }
    uint32_t hv[P], hj = 0;  // head codes; the lane-local positions 7 - j, 4 bits each
#pragma unroll
    for (int i = 0; i < P; ++i) {
        hv[i] = (uint32_t)(key[i] >> 32);
        hj |= ((uint32_t)key[i] & 7u) << (4 * i);
    }
    my_id = 0;
    my_code = 0;
    for (int r = 0; r < k; ++r) {
        const uint32_t m = wave_max_u32(hv[0]);
        const int w = (int)__builtin_ctzll(__ballot(hv[0] == m));  // lowest lane with the maximum
        const int id = base + w * P + 7 - (int)(__builtin_amdgcn_readlane(hj, w) & 7u);
        my_id = lane == r ? id : my_id;
        my_code = lane == r ? m : my_code;
        if (lane == w) {
#pragma unroll
            for (int i = 0; i < P - 1; ++i) hv[i] = hv[i + 1];
            hv[P - 1] = 0u;
            hj >>= 4;
        }
    }
}

// Softmax of the selected logits (lanes 0..k-1 hold rank r's code and expert) into ids / wts.
__device__ __forceinline__ void topk_softmax(uint32_t my_code, int my_id, int k, int* ids, float* wts) {
    const int lane = threadIdx.x & 63;
    const float lg = __uint_as_float((my_code & 0x80000000u) ? (my_code & 0x7fffffffu) : ~my_code);
    const float l0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(lg)));  // the maximum
    const float z = lane < k ? expf(lg - l0) : 0.0f;
    float zs = z + xchg<0>(z);
    zs += xchg<1>(zs);
    zs += xchg<2>(zs);  // lanes 0..7 now all hold the sum over lanes 0..7 (k <= 8)
    if (lane < k) {
        ids[lane] = my_id;
        wts[lane] = z / zs;
    }
}

// Distinct experts in order of first appearance (token, then rank); one lane per (t, r) pair.
// Starts and ends with a barrier.
template <int T>
__device__ void build_slots(int k, SlotTable* st, const int* ids, const float* wts) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    __syncthreads();
    if (T == 1) {  // one token: its k experts are distinct, slot r is rank r
        if (tid < k) {
            st->expert[tid] = ids[tid];
            st->ntok[tid] = 1;
            st->tok[tid][0] = 0;
            st->rank[tid][0] = tid;
            st->w[tid][0] = wts[tid];
        }
        if (tid == 0) st->n = k;
    } else if (wv == 0) {
        const int np = T * k, p = lane;
        const bool valid = p < np;
        const int e = valid ? ids[p] : -1;
        int first = p, j = 0, c = 0;  // first pair with this expert, position among them, count
        for (int q = 0; q < np; ++q) {  // pair q's expert, broadcast from lane q
            const bool same = __builtin_amdgcn_readlane(e, q) == e;
            if (same && q < first) first = q;
            if (same && q < p) ++j;
            if (same) ++c;
        }
        const uint64_t firsts = __ballot(valid && j == 0);
        const int slot = __popcll(firsts & ((1ull << first) - 1ull));
        if (valid) {
            if (j == 0) {
                st->expert[slot] = e;
                st->ntok[slot] = c;
            }
            const int t = p / k;
            st->tok[slot][j] = t;
            st->rank[slot][j] = p - t * k;
            st->w[slot][j] = wts[p];
        }
        if (lane == 0) st->n = __popcll(firsts);
    }
    __syncthreads();
}

// One wave per token (waves past the last token loop, on small workgroups).
template <int T, bool AGENT = false>
__device__ void route_finish(const float (&lgv0)[8], const float* logits, int E, int k, SlotTable* st, int* ids,
                             float* wts) {
    const int wv = threadIdx.x >> 6, NW = blockDim.x >> 6;
    for (int t = wv; t < T; t += NW) {
        float lgv[8];
        if (t == wv) {
#pragma unroll
            for (int j = 0; j < 8; ++j) lgv[j] = lgv0[j];
        } else if (AGENT) {
            load_logits8_agent(logits + t * E, E, lgv);
        } else {
            load_logits<8>(logits + t * E, 0, E, lgv);
        }
        uint32_t my_code;
        int my_id;
        wave_topk<8>(lgv, 0, E, k, my_code, my_id);
        topk_softmax(my_code, my_id, k, ids + t * k, wts + t * k);
    }
    build_slots<T>(k, st, ids, wts);
}

// W > 1 waves per token (the workgroup has at least T W waves): each takes the top-k of its
// 64 P experts, then the token's first wave merges the W lists.
template <int T, int W>
__device__ void route_split(const float (&lgv)[8 / W], int E, int k, SlotTable* st, int* ids, float* wts) {
    constexpr int P = 8 / W;
    __shared__ uint32_t cc[T][W * kMaxTopK];  // candidates: order codes (0 = none) and experts
    __shared__ int ci[T][W * kMaxTopK];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, t = wv / W, w = wv % W;
    if (t < T) {
        uint32_t my_code;
        int my_id;
        wave_topk<P>(lgv, w * 64 * P, E, k, my_code, my_id);
        if (lane < kMaxTopK) {
            cc[t][w * kMaxTopK + lane] = lane < k ? my_code : 0u;
            ci[t][w * kMaxTopK + lane] = my_id;
        }
    }
    __syncthreads();
    if (t < T && w == 0) {
        uint32_t code = lane < W * kMaxTopK ? cc[t][lane] : 0u;
        const int cid = lane < W * kMaxTopK ? ci[t][lane] : 0;
        int my_id = 0;
        uint32_t my_code = 0;
        for (int r = 0; r < k; ++r) {
            const uint32_t m = wave_max_u32(code);
            const int win = (int)__builtin_ctzll(__ballot(code == m));  // lowest (wave, rank) with it
            const int id = __builtin_amdgcn_readlane(cid, win);
            my_id = lane == r ? id : my_id;
            my_code = lane == r ? m : my_code;
            if (lane == win) code = 0u;
        }
        topk_softmax(my_code, my_id, k, ids + t * k, wts + t * k);
    }
    build_slots<T>(k, st, ids, wts);
}

// ------------------------------------------------------------------------------------------------
// 3-4 tokens: the layer's MoE input once per layer (k0), and the FP8 requantisation of every
// routed h vector once per layer (kq) instead of in every down workgroup
// ------------------------------------------------------------------------------------------------

struct K0Args {
    const uint16_t* x;  // [T][H] residual x_l
    uint16_t* xn;       // [T][H] MoE input (bf16)
    uint8_t* xq;        // [T][H] its FP8 codes
    float* xs;          // [T] their scales
    uint16_t* trace;    // [T][H] or null
    float* x_scale;     // [T] or null
    uint8_t* x_codes;   // [T][H] or null
    int H, normalize;
    unsigned long long* stamp;  // timing record of this launch, or null
};

// One workgroup per token (H/4 <= 1024 quads: one load per thread).
template <bool STAMP = false>
__global__ __launch_bounds__(1024) void k0_input(K0Args a) {
    stamp_start<STAMP>(a.stamp);
    extern __shared__ uint4 smem0[];
    __shared__ double redd[16];
    __shared__ float redf[16];
    const int t = blockIdx.x;
    const size_t o = (size_t)t * MOE_SHAPE(H, a.H);
    norm_quant<1>(a.x + o, MOE_SHAPE(H, a.H), MOE_SHAPE(NORM, a.normalize) != 0, (uint16_t*)smem0, a.xn + o, a.xq + o, a.xs + t,
                  a.trace ? a.trace + o : nullptr, a.x_scale ? a.x_scale + t : nullptr,
                  a.x_codes ? a.x_codes + o : nullptr, redd, redf);
    stamp_end<STAMP>(a.stamp);
}

struct KQArgs {
    const float* h;      // [pairs][I]
    const float* hamax;  // [pairs][I/16]
    uint8_t* hq;         // [pairs][I] FP8 codes
    float* hs;           // [pairs] scales
    int I;
    unsigned long long* stamp;  // timing record of this launch, or null
};

// One workgroup per h row (token, rank r <= k; r = k is the shared expert): s_h = max|h| / 448
// (1 when h = 0) from the tile maxima, codes = RNE(h / s_h).
template <bool STAMP = false>
__global__ __launch_bounds__(256) void kq_requant(KQArgs a) {
    stamp_start<STAMP>(a.stamp);
    __shared__ float s;
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int I = MOE_SHAPE(I, a.I), tiles = I / kGuOut, Ih = I / 2;
    float2 v[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int q = tid + c * 256;
        if (q < Ih) v[c] = *(const float2*)(a.h + (size_t)row * I + 2 * q);
    }
    if (tid < 64) {
        float m = 0.0f;
        for (int tl = lane; tl < tiles; tl += 64) m = fmaxf(m, a.hamax[(size_t)row * tiles + tl]);
        m = max64(m);
        if (lane == 0) {
            s = m > 0.0f ? m / 448.0f : 1.0f;
            a.hs[row] = s;
        }
    }
    __syncthreads();
    const float sv = s;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int q = tid + c * 256;
        if (q < Ih) ((uint16_t*)(a.hq + (size_t)row * I))[q] = (uint16_t)e4m3_pack2(v[c].x / sv, v[c].y / sv);
    }
    for (int q = tid + 512; q < Ih; q += 256) {  // wider expert widths
        const float2 w = *(const float2*)(a.h + (size_t)row * I + 2 * q);
        ((uint16_t*)(a.hq + (size_t)row * I))[q] = (uint16_t)e4m3_pack2(w.x / sv, w.y / sv);
    }
    stamp_end<STAMP>(a.stamp);
}

// ------------------------------------------------------------------------------------------------
// k1: router rows (+ the layer's MoE input, stored once for the gate/up kernel)
// ------------------------------------------------------------------------------------------------

struct K1Args {
    const uint16_t* router;  // [E][H]
    const uint16_t* x;       // [T][H] residual x_l (or the MoE input)
    const uint16_t* xn;      // 3-4 tokens: [T][H] MoE input from the input kernel
    uint8_t* xq;             // 1-2 tokens: [T][H] FP8 codes of the MoE input (stored here, shared out)
    float* xs;               // 1-2 tokens: [T] their scales
    uint16_t* trace;         // 1-2 tokens: [T][H] copy of x, or null (workgroup 0)
    float* x_scale;          // 1-2 tokens: [T] or null
    uint8_t* x_codes;        // 1-2 tokens: [T][H] or null
    float* logits;           // [T][E]
    // above gu_route_max_t tokens: the last router workgroup to finish takes the top-k once for the layer
    unsigned* ticket;        // arrivals of router workgroups; zero between layers
    SlotTable* slots_out;    // routed experts of this layer
    int32_t* ids_out;        // [T][k] or null
    float* w_out;            // [T][k] or null
    // 3-4 tokens: workgroups from n_router_wg on compute the shared expert's gate/up items (CUs the
    // router leaves idle), which keeps the gate/up kernel within one workgroup round
    const uint4* w13;
    const uint8_t* w13s;
    float* h;                // [pairs][I]
    float* hamax;            // [pairs][I/16]
    int H, E, k, S, I, normalize, n_router_wg;
    int ntok;                // = T, at run time (keeps the shared expert's token loop a loop)
    unsigned long long* stamp;  // timing record of this launch, or null
};

// One expert row per wave: lane reads 16-byte units lane, lane + 64, ... of the row; bf16 x bf16
// products in fp32 FMA, one logit per wave and token.  At 1-2 tokens every workgroup also
// normalises the input and stores the FP8 codes of its share of it.
template <int T, int BPL, bool MF = false, bool STAMP = false>
__global__ __launch_bounds__(320) void k1_router(K1Args a) {
    stamp_start<STAMP>(a.stamp);
    extern __shared__ uint4 smem1[];
    uint16_t* xb = (uint16_t*)smem1;  // [T][H] bf16 MoE input
    __shared__ double red_d[kMaxWaves * T];
    __shared__ float wmax[kMaxWaves * T];
    __shared__ SlotTable st;
    __shared__ int ids[T * kMaxTopK];
    __shared__ float wts[T * kMaxTopK];
    __shared__ int is_last;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, NW = blockDim.x >> 6;
    const int H = MOE_SHAPE(H, a.H), NU = H / 8;
    // 3-4 tokens: the MoE input comes from the input kernel (once per layer) instead of being
    // recomputed by every workgroup (its fp64 work grows with the token count)
    constexpr bool CENTRAL = T >= 3;
    constexpr bool TICKET = T > gu_route_max_t(MF);  // the last router workgroup takes the top-k
    if constexpr (CENTRAL) {
        if ((int)blockIdx.x >= a.n_router_wg) {  // the shared expert's gate/up items
            __shared__ float red[kMaxWaves * T * kGuRows];
            __shared__ float sx[T];
            const int tiles = MOE_SHAPE(I, a.I) / kGuOut, NC = H / 8, b = blockIdx.x - a.n_router_wg;
            // VALU form: one item per tile and token (a one-token dot reads a quarter of the LDS
            // activations of a 4-token one); the T items of a tile sit 8 apart in blockIdx, on one XCD
            // (whose L2 then serves the tile's weights to all of them) when tiles % 8 == 0
            constexpr bool SPLIT = !MF;
            const int g = tiles % 8 == 0 ? 8 : 1, grp = b / (g * T), r = b - grp * g * T;
            const int tile = SPLIT ? grp * g + r % g : b, t0 = SPLIT ? r / g : 0, ntk = SPLIT ? 1 : a.ntok;
            uint2 xc[T];
            const int xi = min(tid, NC - 1) * 8;
#pragma unroll
            for (int t = 0; t < T; ++t) xc[t] = *(const uint2*)(a.xq + (size_t)t * H + xi);
            const float sxv = a.xs[tid < T ? tid : 0];
            GuLoads<BPL> L;
            L.template issue<MF>(a.w13, a.w13s, MOE_SHAPE(E, a.E), tile, tiles, NW);
            if (tid < T) sx[tid] = sxv;
#pragma unroll
            for (int t = 0; t < T; ++t)
                if (tid < NC) store_codes<MF>(smem1, H, t, tid, xc[t]);
            __syncthreads();
            int tok[T], pair[T];
#pragma unroll
            for (int j = 0; j < T; ++j) {
                tok[j] = min(t0 + j, T - 1);
                pair[j] = tok[j] * (MOE_SHAPE(K, a.k) + MOE_SHAPE(S, a.S)) + MOE_SHAPE(K, a.k);
            }
            gateup_tile<T, BPL, MF>(L, smem1, H, sx, ntk, tok, pair, tile, MOE_SHAPE(I, a.I), a.h, a.hamax, red);
            stamp_end<STAMP>(a.stamp);
            return;
        }
    }
    const int e = blockIdx.x * NW + wv;
    // 1-2 tokens: x first, so that waiting for it does not wait for the router rows
    uint4 xv[T];
    if constexpr (!CENTRAL) moe_input_load<T>(a.x, H, xv);
    __builtin_amdgcn_sched_barrier(0);
    uint4 wr[kMaxWaves];
    {
        const uint4* p = (const uint4*)(a.router + (size_t)min(e, MOE_SHAPE(E, a.E) - 1) * H);
#pragma unroll
        for (int j = 0; j < kMaxWaves; ++j) wr[j] = ld_nt(p + min(lane + 64 * j, NU - 1));
    }
    if constexpr (CENTRAL) {
        for (int i = tid; i < T * NU; i += blockDim.x) ((uint4*)xb)[i] = ((const uint4*)a.xn)[i];
        __syncthreads();
    } else {
        float sx[T];
        moe_input_finish<T>(xv, H, MOE_SHAPE(NORM, a.normalize) != 0, xb, red_d, wmax, sx);
        if (blockIdx.x == 0 && a.trace)
            for (int i = tid; i < T * NU; i += blockDim.x) ((uint4*)a.trace)[i] = ((const uint4*)a.x)[i];
        quantize_slice<T>(xb, H, sx, a.xq, a.xs, a.x_codes, a.x_scale);
    }
    if (e < MOE_SHAPE(E, a.E)) {
        float acc[T];
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t] = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxWaves; ++j) {
            const int u = lane + 64 * j;
            if (u < NU) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const uint4 xv = *(const uint4*)(xb + t * H + u * 8);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t d = comp(wr[j], q), xx = comp(xv, q);
                        acc[t] = fmaf(__uint_as_float(d << 16), __uint_as_float(xx << 16), acc[t]);
                        acc[t] = fmaf(__uint_as_float(d & 0xffff0000u), __uint_as_float(xx & 0xffff0000u), acc[t]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the LDS reads of later units from being hoisted
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float v = sum64(acc[t]);
            if (lane == 0) {
                if constexpr (TICKET)  // write-through: the last workgroup reads it without a cache flush
                    __hip_atomic_store(a.logits + t * MOE_SHAPE(E, a.E) + e, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                else
                    a.logits[t * MOE_SHAPE(E, a.E) + e] = v;
            }
        }
    }
    if constexpr (TICKET) {
        // Above gu_route_max_t tokens: the last router workgroup to arrive takes the top-k of every token
        // (the gate/up workgroups would otherwise each redo it for all tokens).  Ordering rests on the ISA, not on
        // release/acquire (whose L2 write-back in every workgroup costs microseconds): the logits are
        // agent-scope atomic stores, written through to the device-coherent level; vmcnt(0) waits
        // until the memory has acknowledged them, before the barrier and the arrival; the last
        // workgroup reads them with agent-scope atomic loads, which do not hit in the non-coherent L2.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if (tid == 0)
            is_last = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                      (unsigned)(a.n_router_wg - 1);
        __syncthreads();
        if (is_last) {
            float lgv[8];
            load_logits8_agent(a.logits + min(wv, T - 1) * MOE_SHAPE(E, a.E), MOE_SHAPE(E, a.E), lgv);
            route_finish<T, true>(lgv, a.logits, MOE_SHAPE(E, a.E), MOE_SHAPE(K, a.k), &st, ids, wts);
            for (int i = tid; i < (int)(sizeof(SlotTable) / 4); i += blockDim.x)
                ((int*)a.slots_out)[i] = ((const int*)&st)[i];
            for (int i = tid; i < T * MOE_SHAPE(K, a.k); i += blockDim.x) {
                if (a.ids_out) a.ids_out[i] = ids[i];
                if (a.w_out) a.w_out[i] = wts[i];
            }
            if (tid == 0) *a.ticket = 0u;  // read again only by the next layer's router, after this kernel
        }
    }
    stamp_end<STAMP>(a.stamp);
}

// ------------------------------------------------------------------------------------------------
// k2: top-k (redone by every routed workgroup) + gate/up tiles of the routed and shared experts
// ------------------------------------------------------------------------------------------------

struct K2Args {
    const float* logits;     // [T][E]
    const uint8_t* xq;       // [T][H] FP8 codes of the MoE input
    const float* xs;         // [T] their scales
    const uint4* w13;
    const uint8_t* w13s;
    float* h;                // [pairs][I]
    float* hamax;            // [pairs][I/16]
    SlotTable* slots;        // routed experts of this layer: stored here for the down kernel (up to
                             // gu_route_max_t tokens) or read (above, from the router kernel)
    int32_t* ids_out;        // [T][k] or null
    float* w_out;            // [T][k] or null
    int H, E, k, S, I, n_sh_wg;
    int ntok;                // = T, at run time (keeps the shared expert's token loop a loop)
    unsigned long long* stamp;  // timing record of this launch, or null
};

// Workgroups [0, n_sh_wg): the shared expert's gate/up tiles for every token (no routing needed).
// The others: workgroup (slot, tile) takes the top-k of every token from the logits (one wave per
// token), builds the distinct-expert list, and computes tile `tile` of routed expert `slot` for the
// tokens routed to it (slots beyond the list exit).  The first of them stores the list, the ids and
// the weights.
// VALU form with the router kernel's top-k (4 tokens): at most 64 VGPRs, six workgroups per CU, so
// that the 4-token grid of 32 slots x 48 tiles runs in one round (44.1 against 44.7 us/layer).  The
// stamping instance is left uncapped (under the cap its stamps cost it six VGPR spills): it runs
// five workgroups per CU, so the timing record overstates this kernel slightly at 4 tokens.
template <int T, int BPL, int W, bool MF = false, bool STAMP = false>
__global__ __launch_bounds__(320)
__attribute__((amdgpu_waves_per_eu(T > gu_route_max_t(MF) && !MF && !STAMP ? 8 : 1)))
void k2_gateup(K2Args a) {
    stamp_start<STAMP>(a.stamp);
    extern __shared__ uint4 smem2[];
    // smem2: the input's FP8 codes as f16 pairs [T][H/2], or as bf16 [T][H] (MF)
    __shared__ float red[kMaxWaves * T * kGuRows];
    __shared__ float sx[T];
    __shared__ SlotTable st;
    __shared__ int ids[T * kMaxTopK];
    __shared__ float wts[T * kMaxTopK];
    const int tid = threadIdx.x, NW = blockDim.x >> 6;
    const int H = MOE_SHAPE(H, a.H), I = MOE_SHAPE(I, a.I), k = MOE_SHAPE(K, a.k), tiles = I / kGuOut, NC = H / 8;
    const bool is_shared = (int)blockIdx.x < a.n_sh_wg;

    // the input's FP8 codes, loaded first (one 8-byte load per thread and token), then the logits
    uint2 xc[T];
    const int xi = min(tid, NC - 1) * 8;  // loads unconditional (clamped), stores guarded
#pragma unroll
    for (int t = 0; t < T; ++t) xc[t] = *(const uint2*)(a.xq + (size_t)t * H + xi);
    const float sxv = a.xs[tid < T ? tid : 0];
    // up to gu_route_max_t tokens every routed workgroup takes the top-k itself; above, the router kernel did
    constexpr bool ROUTE = T <= gu_route_max_t(MF);
    // W waves per token take the top-k together (W = 1: one wave per token)
    float lgv[8 / W];
    if constexpr (ROUTE) route_issue<T, W>(a.logits, MOE_SHAPE(E, a.E), lgv);  // shared workgroups load them too: exact waits below

    // the codes' f16 (bf16) values into LDS while the logits are in flight
    if (tid < T) sx[tid] = sxv;
#pragma unroll
    for (int t = 0; t < T; ++t)
        if (tid < NC) store_codes<MF>(smem2, H, t, tid, xc[t]);

    GuLoads<BPL> L;
    int tok[T], pair[T], nt, tile;
    if (is_shared) {
        tile = blockIdx.x;
        L.template issue<MF>(a.w13, a.w13s, MOE_SHAPE(E, a.E), blockIdx.x, tiles, NW);
        nt = a.ntok;
#pragma unroll
        for (int j = 0; j < T; ++j) {
            tok[j] = j;
            pair[j] = j * (k + MOE_SHAPE(S, a.S)) + k;
        }
    } else {
        const int b = blockIdx.x - a.n_sh_wg, slot = b / tiles;
        tile = b - slot * tiles;
        if constexpr (ROUTE) {
            if constexpr (W > 1)
                route_split<T, W>(lgv, MOE_SHAPE(E, a.E), k, &st, ids, wts);
            else
                route_finish<T>(lgv, a.logits, MOE_SHAPE(E, a.E), k, &st, ids, wts);
            if (b == 0) {  // the first routed workgroup publishes the routing of the layer
                for (int i = tid; i < (int)(sizeof(SlotTable) / 4); i += blockDim.x)
                    ((int*)a.slots)[i] = ((const int*)&st)[i];
                for (int i = tid; i < T * k; i += blockDim.x) {
                    if (a.ids_out) a.ids_out[i] = ids[i];
                    if (a.w_out) a.w_out[i] = wts[i];
                }
            }
        }
        // the slot's entries: from LDS (routed here) or straight from the stored list (uniform loads)
        const SlotTable& sl = ROUTE ? st : *a.slots;
        if (slot >= sl.n) {  // no expert for this slot: the whole workgroup leaves
            if constexpr (STAMP)
                if (threadIdx.x == 0) a.stamp[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
            return;
        }
        L.template issue<MF>(a.w13, a.w13s, sl.expert[slot], tile, tiles, NW);
        nt = sl.ntok[slot];
#pragma unroll
        for (int j = 0; j < T; ++j) {
            const bool on = j < nt;
            tok[j] = on ? sl.tok[slot][j] : 0;
            pair[j] = on ? sl.tok[slot][j] * (k + MOE_SHAPE(S, a.S)) + sl.rank[slot][j] : 0;
        }
    }
    __syncthreads();
    gateup_tile<T, BPL, MF>(L, smem2, H, sx, nt, tok, pair, tile, I, a.h, a.hamax, red);
    stamp_end<STAMP>(a.stamp);
}

// ------------------------------------------------------------------------------------------------
// k3: routed + shared down rows, combine, residual
// ------------------------------------------------------------------------------------------------

struct K3Args {
    const SlotTable* slots;
    const uint4* w2;
    const uint8_t* w2s;
    const float* h;          // [pairs][I]
    const float* hamax;      // [pairs][I/16]
    const uint8_t* hq;       // [pairs][I] FP8 codes of h (3-4 tokens: from the requantisation kernel)
    const float* hs;         // [pairs] their scales
    const uint16_t* xres;    // [T][H] residual x_l, or null
    uint16_t* xnext;         // [T][H] bf16(x_l + y), or null
    float* y;                // [T][H] or null
    int H, E, k, S, I;
    int rows;                // output rows per workgroup (H / grid)
    int units_max;           // (slot, row) units of the largest layer: (routed slots + S T) * rows
    unsigned long long* stamp;  // timing record of this launch, or null
};

// One workgroup per `rows` consecutive output rows (H / rows = one workgroup per CU, so no CU holds
// two while others hold one).  Work items ("slots") are the distinct routed experts of the layer
// followed by the shared expert once per token (weight 1).  The (slot, row) units are spread over
// the waves, R = 64 / KSUB units per wave and group, KSUB lanes per unit (ITERS blocks of 32 each),
// UPW groups per wave.  Each unit's routing-weighted result goes to LDS and the epilogue sums a
// row's units in slot order.  h vectors are indexed by their row t*(k+S) + r (r = k: shared).
template <int KSUB, int ITERS, int T, int UPW, bool STAMP = false>
__global__ __launch_bounds__(768) void k3_down(K3Args a) {
    stamp_start<STAMP>(a.stamp);
    constexpr int R = kWave / KSUB;  // units per wave and group; rows per repacked tile
    constexpr bool CODES = T >= kKqMinT;  // FP8 h codes from the requantisation kernel
    constexpr int MAXP = CODES ? 1 : T == 1 ? 5 : 9;  // h columns (rows of h) per thread, loaded up front
    extern __shared__ uint4 smem3[];
    const int H = MOE_SHAPE(H, a.H), I = MOE_SHAPE(I, a.I), k = MOE_SHAPE(K, a.k), Ih = I / 2, tiles = I / kGuOut, rtiles = H / R;
    const int nrows = T * (k + MOE_SHAPE(S, a.S));
    half2_t* hh = (half2_t*)smem3;                     // [T*(k+S)][I/2] f16 values of h's FP8 codes
    float* red = (float*)(hh + (size_t)nrows * Ih);    // [units][T] routing-weighted unit results
    __shared__ float s_h[kMaxPairs];
    __shared__ SlotTable s_st;  // copy of the routed slots
    const int tid = threadIdx.x, nth = blockDim.x, lane = tid & 63, wv = tid >> 6, NW = nth >> 6;
    const int RW = a.rows, row0 = blockIdx.x * RW, ks = lane % KSUB;
    // epilogue operand of this thread's output element (row row0 + tid % RW, token tid / RW)
    const int oe = tid < RW * T ? tid : 0;
    const size_t oo = (size_t)(oe / RW) * H + row0 + oe % RW;
    const uint16_t xr_pre = a.xnext ? a.xres[oo] : (uint16_t)0;
    // thread -> (column pair q, row group g); G groups cover the rows g, g + G, ...
    const int G = nth / Ih, q0 = tid % Ih, g0 = tid / Ih;
    const bool loader = !CODES && G > 0 && g0 < G;

    // 1. independent loads, all issued before any is used: slot list, tile maxima of this wave's
    // rows (row = wave + m * waves), h of every row (first MAXP * G rows).  Indices are clamped
    // instead of branched on, so that the waits below stay exact.
    constexpr int NSU = (int)(sizeof(SlotTable) / 16);  // 16-byte units of the slot list
    static_assert(sizeof(SlotTable) % 16 == 0 && NSU <= 128, "slot list: one unit per thread of two waves");
    const uint4 stu = ((const uint4*)a.slots)[min(tid, NSU - 1)];
    float hm[4];
    if constexpr (!CODES) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int p = min(wv + NW * m, nrows - 1);
            hm[m] = a.hamax[(size_t)p * tiles + min(lane, tiles - 1)];
        }
    }
    float2 hv[MAXP];
    if constexpr (!CODES) {
        const int qc = min(q0, Ih - 1);
#pragma unroll
        for (int m = 0; m < MAXP; ++m) hv[m] = *(const float2*)(a.h + (size_t)min(g0 + m * G, nrows - 1) * I + 2 * qc);
    }
    // 3-4 tokens: the h codes (16 per unit) and scales
    constexpr int HQ = CODES ? 3 : 1;  // code units per thread loaded up front
    const int nq = nrows * (I / 16);
    uint4 hqv[HQ];
    float hsv = 0.0f;
    if constexpr (CODES) {
#pragma unroll
        for (int m = 0; m < HQ; ++m) hqv[m] = *(const uint4*)(a.hq + (size_t)min(tid + m * nth, nq - 1) * 16);
        hsv = a.hs[min(tid, nrows - 1)];
    }
    if (tid < NSU) ((uint4*)&s_st)[tid] = stu;
    __syncthreads();
    const int n = s_st.n, nall = n + MOE_SHAPE(S, a.S) * T, nunits = nall * RW;  // routed slots, then shared per token

    // 2. down weight loads of this wave's units: unit u = (wave + NW m) R + lane / KSUB is slot
    // u / RW, row row0 + u % RW (units past the last repeat it; their results are not stored).
    // With KSUB = 8 the unit's ITERS x 8 scale bytes come in as one dword per lane (lanes
    // ks < 2 ITERS) and are handed to their lanes by ds_bpermute: one load instead of ITERS.
    static_assert(KSUB != 8 || ITERS <= 4, "scale bytes of a unit: one dword per lane");
    uint4 wr[UPW][ITERS];
    uint32_t sw[UPW][KSUB == 8 ? 1 : ITERS];
#pragma unroll
    for (int m = 0; m < UPW; ++m) {
        const int u = min((wv + NW * m) * R + lane / KSUB, nunits - 1);
        const int s = u / RW, r = row0 + (u - s * RW);
        const int ex = s < n ? s_st.expert[s] : MOE_SHAPE(E, a.E);
        const size_t tb = ((size_t)ex * rtiles + r / R) * ITERS;  // first 1 KiB unit of the row's tile
        const int lo = (r % R) * KSUB + ks;
#pragma unroll
        for (int it = 0; it < ITERS; ++it) wr[m][it] = ld_nt(a.w2 + (tb + it) * kWave + lo);
        if constexpr (KSUB == 8) {
            const int j = ks % (2 * ITERS);  // dword j: iteration j / 2, half j % 2
            sw[m][0] = __builtin_nontemporal_load(
                (const uint32_t*)(a.w2s + (tb + j / 2) * kWave + (size_t)(r % R) * KSUB) + (j & 1));
        } else {
#pragma unroll
            for (int it = 0; it < ITERS; ++it) sw[m][it] = __builtin_nontemporal_load(a.w2s + (tb + it) * kWave + lo);
        }
    }

    // 3. FP8 requantisation of every h row into LDS (or the decode of its codes)
    if constexpr (CODES) {
        // unit i of h's codes (16 codes) -> 8 f16 pairs at hh + 8 i (rows of I/16 units are contiguous)
#pragma unroll
        for (int m = 0; m < HQ; ++m) {
            const int i = tid + m * nth;
            if (i < nq) {
                half2_t* o = hh + (size_t)i * 8;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    o[2 * q] = e4m3x2_to_f16x2(comp(hqv[m], q) & 0xffffu);
                    o[2 * q + 1] = e4m3x2_to_f16x2(comp(hqv[m], q) >> 16);
                }
            }
        }
        for (int i = tid + HQ * nth; i < nq; i += nth) {  // more units than threads can preload
            const uint4 cw = *(const uint4*)(a.hq + (size_t)i * 16);
            half2_t* o = hh + (size_t)i * 8;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o[2 * q] = e4m3x2_to_f16x2(comp(cw, q) & 0xffffu);
                o[2 * q + 1] = e4m3x2_to_f16x2(comp(cw, q) >> 16);
            }
        }
        if (tid < nrows) s_h[tid] = hsv;
        __syncthreads();
    } else {
        for (int m = 0; m < 4 && wv + NW * m < nrows; ++m) {  // uniform per wave
            const float mx = max64(lane < tiles ? hm[m] : 0.0f);
            if (lane == 0) s_h[wv + NW * m] = mx > 0.0f ? mx / 448.0f : 1.0f;
        }
        for (int p = wv + 4 * NW; p < nrows; p += NW) {  // more rows than 4 per wave (small grids)
            float v = 0.0f;
            for (int tl = lane; tl < tiles; tl += 64) v = fmaxf(v, a.hamax[(size_t)p * tiles + tl]);
            const float mx = max64(v);
            if (lane == 0) s_h[p] = mx > 0.0f ? mx / 448.0f : 1.0f;
        }
        __syncthreads();
        if (loader) {
#pragma unroll
            for (int m = 0; m < MAXP; ++m) {
                const int p = g0 + m * G;
                if (p < nrows) hh[p * Ih + q0] = e4m3x2_to_f16x2(e4m3_pack2(hv[m].x / s_h[p], hv[m].y / s_h[p]));
            }
        }
        // rows beyond the up-front batch, or every row when there are fewer threads than columns
        const int p0 = G > 0 ? (G * MAXP < nrows ? G * MAXP : nrows) : 0;
        for (int i = tid; i < (nrows - p0) * Ih; i += nth) {
            const int p = p0 + i / Ih, q = i % Ih;
            const float2 v = *(const float2*)(a.h + (size_t)p * I + 2 * q);
            hh[p * Ih + q] = e4m3x2_to_f16x2(e4m3_pack2(v.x / s_h[p], v.y / s_h[p]));
        }
        __syncthreads();
    }

    // 4. block dot products of each unit, routing-weighted per token, reduced over the unit's lanes
#pragma unroll
    for (int m = 0; m < UPW; ++m) {
        const int u0 = (wv + NW * m) * R + lane / KSUB, u = min(u0, nunits - 1);
        const int s = u / RW;
        const bool shs = s >= n;  // the shared expert for token s - n: rank k, weight 1
        const int si = min(s, kMaxSlots - 1), ts = s - n;
        const int nt = shs ? 1 : s_st.ntok[si];
        int pp[T];
#pragma unroll
        for (int j = 0; j < T; ++j)
            pp[j] = j < nt ? (shs ? ts * (k + MOE_SHAPE(S, a.S)) + k : s_st.tok[si][j] * (k + MOE_SHAPE(S, a.S)) + s_st.rank[si][j]) : 0;
        float pj[T];
#pragma unroll
        for (int j = 0; j < T; ++j) pj[j] = 0.0f;
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            uint32_t sbyte;
            if constexpr (KSUB == 8) {
                const uint32_t sd = (uint32_t)__builtin_amdgcn_ds_bpermute(
                    ((lane & ~7) + 2 * it + (ks >> 2)) * 4, (int)sw[m][0]);
                sbyte = sd >> (8 * (ks & 3));
            } else {
                sbyte = sw[m][it];
            }
            const float scale = e8m0_to_f32(sbyte & 0xffu);
            const int pbase = (it * KSUB + ks) * (kBlock / 2);
            const half2_t* xp[T];
#pragma unroll
            for (int j = 0; j < T; ++j) xp[j] = hh + pp[j] * Ih + pbase;
            float q[T];
#pragma unroll
            for (int j = 0; j < T; ++j) q[j] = 0.0f;
            block_dot_nt<T>(wr[m][it], xp, q, nt);
#pragma unroll
            for (int j = 0; j < T; ++j) pj[j] = fmaf(q[j], scale, pj[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        float v[T];
#pragma unroll
        for (int t = 0; t < T; ++t) v[t] = 0.0f;
#pragma unroll
        for (int j = 0; j < T; ++j) {
            if (j < nt) {
                const int tk = shs ? ts : s_st.tok[si][j];
                const float cf = (shs ? 1.0f : s_st.w[si][j]) * s_h[pp[j]];
#pragma unroll
                for (int t = 0; t < T; ++t)
                    if (t == tk) v[t] = fmaf(cf, pj[j], v[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < T; ++t) v[t] = sum_ksub<KSUB>(v[t]);
        if (ks == 0 && u0 < nunits) {
#pragma unroll
            for (int t = 0; t < T; ++t) red[u0 * T + t] = v[t];
        }
    }
    __syncthreads();

    // 5. each output row: its units summed in slot order (routed slots, then shared)
    for (int idx = tid; idx < RW * T; idx += nth) {
        const int t = idx / RW, r = idx - t * RW;
        float ysum = 0.0f;
        for (int s = 0; s < nall; ++s) ysum += red[(s * RW + r) * T + t];
        const size_t o = (size_t)t * H + row0 + r;
        if (a.y) a.y[o] = ysum;
        if (a.xnext) a.xnext[o] = f32_to_bf16(bf16_to_f32(idx == tid ? xr_pre : a.xres[o]) + ysum);
    }
    stamp_end<STAMP>(a.stamp);
}

MOE_KERNELS_NS_END
