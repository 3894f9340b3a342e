// moe_kernels.hip -- gfx950 kernels of the W4A8 sparse-MoE decode step.
//
// One layer is three launches on the caller's stream:
//   router_kernel  bf16 router GEMV, split over (K slice, 64-row tile) workgroups; the last
//                  workgroup to finish (atomic ticket) sums the partial logits, takes the top-k
//                  per token in one wavefront (lower index first on ties), computes the softmax
//                  weights and writes the list of distinct experts ("slots") of this call.
//   gateup_kernel  one workgroup per (32-row h tile, slot): streams the MXFP4 gate and up rows,
//                  dequantises E2M1 codes to f16 pairs in VGPRs, dot2 with the FP8-quantised
//                  activation held in LDS, and writes h = SiLU(gate) * up plus the tile's max |h|.
//   down_kernel    one workgroup per output-row tile, all experts: requantises every (slot,
//                  token) h vector to FP8 in LDS, streams the MXFP4 down rows of every slot and
//                  sums the routing-weighted results in a fixed order (no float atomics), then
//                  writes y and the updated bf16 residual.
//
// What is computed follows the MoE decode step described on the pages (tanhow.com, "NVIDIA 在单台
// DGX Spark 上叠加三项优化..." sections "Ling 3.0 是什么" (8 of 512 routed experts + 1 shared) and
// "三项优化是什么" items 1 and 3 (width-768 MXFP4 experts; a 4-position verify touching up to 32
// experts); devotd.net "dgx-spark-moe-inference-optimizations" section 2 (MXFP4 = blocked 4-bit
// float, 4-bit weights with 8-bit activations)).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_launch.h"

namespace moe {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------------------------------
// small helpers
// ------------------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// E8M0 byte -> fp32 2^(b-127) by placing b in the fp32 exponent field (exact for 1 <= b <= 254).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) { return __uint_as_float((b & 0xffu) << 23); }

// Two fp32 values -> two OCP E4M3 codes (round to nearest even) in the low 16 bits.
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) 128-bit and 64-bit loads of weights that are read once per pass.
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt(const uint2* p) {
    const u32x2 v = __builtin_nontemporal_load((const u32x2*)p);
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ __forceinline__ uint32_t comp(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
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

__device__ __forceinline__ float wave_max(float v, int width) {
    for (int off = width >> 1; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, width));
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ------------------------------------------------------------------------------------------------
// repack kernels (canonical row-major -> lane tiles; pure permutations of 16-byte units / bytes)
// ------------------------------------------------------------------------------------------------

__global__ void repack_router(const uint16_t* __restrict__ src, uint4* __restrict__ dst, int E, int H, int RT) {
    const int NU = H / kRouterUnitElems;
    const uint64_t total = (uint64_t)RT * NU * kWave;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        const uint64_t r1 = u / kWave;
        const int unit = (int)(r1 % NU);
        const int rt = (int)(r1 / NU);
        const int row = rt * kRouterRows + lane;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < E) v = *(const uint4*)(src + (uint64_t)row * H + (uint64_t)unit * kRouterUnitElems);
        dst[u] = v;
    }
}

__global__ void repack_w13(const uint4* __restrict__ src, uint4* __restrict__ dst, int nexp, int I, int H) {
    const int NB = H / kBlock, tiles = I / kGuHalf;
    const uint64_t total = (uint64_t)nexp * tiles * NB * kWave;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        const uint64_t r1 = u / kWave;
        const int c = (int)(r1 % NB);
        const uint64_t r2 = r1 / NB;
        const int tile = (int)(r2 % tiles);
        const uint64_t e = r2 / tiles;
        const int row = lane < kGuHalf ? tile * kGuHalf + lane : I + tile * kGuHalf + lane - kGuHalf;
        dst[u] = src[(e * 2 * I + row) * NB + c];
    }
}

__global__ void repack_w13s(const uint8_t* __restrict__ src, uint2* __restrict__ dst, int nexp, int I, int H) {
    const int NB = H / kBlock, NG = NB / kGuBlocksPerWave, tiles = I / kGuHalf;
    const uint64_t total = (uint64_t)nexp * tiles * NG * kWave;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        const uint64_t r1 = u / kWave;
        const int g = (int)(r1 % NG);
        const uint64_t r2 = r1 / NG;
        const int tile = (int)(r2 % tiles);
        const uint64_t e = r2 / tiles;
        const int row = lane < kGuHalf ? tile * kGuHalf + lane : I + tile * kGuHalf + lane - kGuHalf;
        dst[u] = *(const uint2*)(src + (e * 2 * I + row) * NB + g * kGuBlocksPerWave);
    }
}

__global__ void repack_w2(const uint4* __restrict__ src, uint4* __restrict__ dst, int nexp, int H, int I, int ksub) {
    const int NB = I / kBlock, R = kWave / ksub, iters = NB / ksub, tiles = H / R;
    const uint64_t total = (uint64_t)nexp * tiles * iters * kWave;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        const uint64_t r1 = u / kWave;
        const int it = (int)(r1 % iters);
        const uint64_t r2 = r1 / iters;
        const int tile = (int)(r2 % tiles);
        const uint64_t e = r2 / tiles;
        const int row = tile * R + lane / ksub;
        const int c = it * ksub + lane % ksub;
        dst[u] = src[(e * H + row) * NB + c];
    }
}

__global__ void repack_w2s(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int nexp, int H, int I, int ksub) {
    const int NB = I / kBlock, R = kWave / ksub, iters = NB / ksub, tiles = H / R;
    const uint64_t total = (uint64_t)nexp * tiles * iters * kWave;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        const uint64_t r1 = u / kWave;
        const int it = (int)(r1 % iters);
        const uint64_t r2 = r1 / iters;
        const int tile = (int)(r2 % tiles);
        const uint64_t e = r2 / tiles;
        const int row = tile * R + lane / ksub;
        const int c = it * ksub + lane % ksub;
        dst[u] = src[(e * H + row) * NB + c];
    }
}

// ------------------------------------------------------------------------------------------------
// router GEMV + top-k + softmax + slot list
// ------------------------------------------------------------------------------------------------

struct RouterArgs {
    const uint4* w;         // repacked router of this layer
    const uint16_t* x;      // [T][H] residual x_l (or the MoE input when normalize == 0)
    uint16_t* xin;          // [T][H] MoE input, written by the rt == 0 workgroups
    uint16_t* trace;        // [T][H] copy of x, or null
    float* partial;         // [G][T][RT*64]
    unsigned* ticket;       // zero between calls
    SlotTable* slots;
    int32_t* ids_out;       // [T][k] or null
    float* w_out;           // [T][k] or null
    int H, E, k, S, normalize;
};

template <int T>
__device__ void router_finish(const RouterArgs& a, int G, int RT) {
    __shared__ float lg[T][512];
    __shared__ int s_ids[T][kMaxTopK];
    __shared__ float s_lv[T][kMaxTopK];
    __shared__ float s_w[T][kMaxTopK];
    __shared__ short slot_of[512];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int E = a.E, k = a.k, Ep = RT * kRouterRows;
    for (int i = tid; i < T * E; i += blockDim.x) {
        const int t = i / E, e = i - t * E;
        float s = 0.0f;
        for (int g = 0; g < G; ++g) s += __builtin_nontemporal_load(a.partial + ((size_t)g * T + t) * Ep + e);
        lg[t][e] = s;
    }
    for (int i = tid; i < E; i += blockDim.x) slot_of[i] = -1;
    __syncthreads();
    if (wv < T) {
        const int t = wv;
        float v[8];
        unsigned taken = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = lane + 64 * j;
            v[j] = e < E ? lg[t][e] : -INFINITY;
        }
        for (int r = 0; r < k; ++r) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int e = lane + 64 * j;
                if (e < E && !((taken >> j) & 1u) && (v[j] > bv || (v[j] == bv && e < bi))) {
                    bv = v[j];
                    bi = e;
                }
            }
            for (int off = 32; off > 0; off >>= 1) {
                const float ov = __shfl_xor(bv, off, 64);
                const int oi = __shfl_xor(bi, off, 64);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
            if (lane == 0) {
                s_ids[t][r] = bi;
                s_lv[t][r] = bv;
            }
        }
        if (lane == 0) {
            const float m = s_lv[t][0];
            float z[kMaxTopK], Z = 0.0f;
            for (int r = 0; r < k; ++r) {
                z[r] = expf(s_lv[t][r] - m);
                Z += z[r];
            }
            for (int r = 0; r < k; ++r) {
                const float w = z[r] / Z;
                s_w[t][r] = w;
                if (a.ids_out) a.ids_out[t * k + r] = s_ids[t][r];
                if (a.w_out) a.w_out[t * k + r] = w;
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        SlotTable* st = a.slots;
        int n = 0;
        for (int t = 0; t < T; ++t) {
            for (int r = 0; r < k; ++r) {
                const int e = s_ids[t][r];
                int s = slot_of[e];
                if (s < 0) {
                    s = n++;
                    slot_of[e] = (short)s;
                    st->expert[s] = e;
                    st->ntok[s] = 0;
                }
                const int j = st->ntok[s]++;
                st->tok[s][j] = t;
                st->w[s][j] = s_w[t][r];
            }
        }
        if (a.S) {
            const int s = n++;
            st->expert[s] = E;
            st->ntok[s] = T;
            for (int t = 0; t < T; ++t) {
                st->tok[s][t] = t;
                st->w[s][t] = 1.0f;
            }
        }
        st->n = n;
        *a.ticket = 0u;
    }
}

template <int T>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
    __shared__ float xs[T][kRouterSlice];
    __shared__ double red_d[kRouterWaves][T];
    __shared__ float redf[kRouterWaves][T][kWave];
    __shared__ int is_last;
    const int g = blockIdx.x, rt = blockIdx.y, G = gridDim.x, RT = gridDim.y;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int H = a.H, NU = H / kRouterUnitElems;

    // 1. weight loads for this wave's 8 units (64 K elements) of the 64-row tile
    uint4 wr[kRouterUnitsPerWave];
    {
        const uint4* p = a.w + ((size_t)rt * NU + (size_t)g * (kRouterSlice / kRouterUnitElems) +
                                wv * kRouterUnitsPerWave) * kWave + lane;
#pragma unroll
        for (int i = 0; i < kRouterUnitsPerWave; ++i) wr[i] = ld_nt(p + i * kWave);
    }

    // 2. MoE input of this workgroup's K slice: x itself, or bf16(fl32(x * r)) with
    //    r = 1 / sqrt(mean(x^2) + 1e-6) evaluated in fp64
    const int c = g * kRouterSlice + tid;
    double r[T];
    if (a.normalize) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            double ss = 0.0;
            for (int i = tid; i < H; i += blockDim.x) {
                const double v = (double)bf16_to_f32(a.x[(size_t)t * H + i]);
                ss += v * v;
            }
            ss = wave_sum_d(ss);
            if (lane == 0) red_d[wv][t] = ss;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < T; ++t) {
            double ss = 0.0;
            for (int w = 0; w < kRouterWaves; ++w) ss += red_d[w][t];
            r[t] = 1.0 / sqrt(ss / (double)H + 1e-6);
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const uint16_t xb = a.x[(size_t)t * H + c];
        uint16_t ib = xb;
        if (a.normalize) ib = f32_to_bf16((float)((double)bf16_to_f32(xb) * r[t]));
        xs[t][tid] = bf16_to_f32(ib);
        if (rt == 0) {
            a.xin[(size_t)t * H + c] = ib;
            if (a.trace) a.trace[(size_t)t * H + c] = xb;
        }
    }
    __syncthreads();

    // 3. partial logits: fp32 FMA of exact bf16 x bf16 products
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < kRouterUnitsPerWave; ++i) {
        const int k0 = wv * (kRouterUnitsPerWave * kRouterUnitElems) + i * kRouterUnitElems;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t d = comp(wr[i], q);
            const float wlo = __uint_as_float(d << 16), whi = __uint_as_float(d & 0xffff0000u);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                acc[t] = fmaf(wlo, xs[t][k0 + 2 * q], acc[t]);
                acc[t] = fmaf(whi, xs[t][k0 + 2 * q + 1], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) redf[wv][t][lane] = acc[t];
    __syncthreads();
    if (tid < T * kWave) {
        const int t = tid >> 6, l = tid & 63;
        float s = 0.0f;
        for (int w = 0; w < kRouterWaves; ++w) s += redf[w][t][l];
        a.partial[((size_t)g * T + t) * (RT * kRouterRows) + rt * kRouterRows + l] = s;
    }

    // 4. the last workgroup to arrive finishes the routing
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = atomicAdd(a.ticket, 1u) == (unsigned)(G * RT - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    router_finish<T>(a, G, RT);
}

// ------------------------------------------------------------------------------------------------
// gate/up GEMV with fused SiLU(gate) * up
// ------------------------------------------------------------------------------------------------

struct GateUpArgs {
    const uint4* w13;       // repacked codes of this layer
    const uint2* w13s;      // repacked scales
    const uint16_t* xin;    // [T][H] MoE input (bf16)
    const SlotTable* slots;
    float* h;               // [kMaxSlots][kMaxTokens][I]
    float* hamax;           // [kMaxSlots][kMaxTokens][I/32]
    float* x_scale_out;     // [T] or null
    uint8_t* x_codes_out;   // [T][H] or null
    int H, I;
};

template <int T>
__global__ __launch_bounds__(640) void gateup_kernel(GateUpArgs a) {
    extern __shared__ uint4 smem_gu[];
    half2_t* xh = (half2_t*)smem_gu;  // [T][H/2]
    __shared__ float wmax[16][T];
    __shared__ float red[16][T][kWave];
    const int tile = blockIdx.x, slot = blockIdx.y;
    const SlotTable* st = a.slots;
    const int n = st->n;
    if (slot >= n) return;
    const int H = a.H, I = a.I, NB = H / kBlock, tiles = I / kGuHalf, Hh = H / 2;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, NW = blockDim.x >> 6;
    const int e = st->expert[slot], ntok = st->ntok[slot];
    int tok[T];
#pragma unroll
    for (int j = 0; j < T; ++j) tok[j] = j < ntok ? st->tok[slot][j] : 0;

    // 1. weight loads: 8 MX blocks of this lane's row
    uint4 wr[kGuBlocksPerWave];
    const size_t tbase = (size_t)e * tiles + tile;
    {
        const uint4* p = a.w13 + (tbase * NB + (size_t)wv * kGuBlocksPerWave) * kWave + lane;
#pragma unroll
        for (int i = 0; i < kGuBlocksPerWave; ++i) wr[i] = ld_nt(p + i * kWave);
    }
    const uint2 sc = ld_nt(a.w13s + (tbase * (NB / kGuBlocksPerWave) + wv) * kWave + lane);

    // 2. per-token FP8 quantisation of the input into LDS (as exact f16 values)
#pragma unroll
    for (int t = 0; t < T; ++t) {
        float m = 0.0f;
        for (int i = tid; i < H; i += blockDim.x) m = fmaxf(m, fabsf(bf16_to_f32(a.xin[(size_t)t * H + i])));
        m = wave_max(m, 64);
        if (lane == 0) wmax[wv][t] = m;
    }
    __syncthreads();
    float sx[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        float m = 0.0f;
        for (int w = 0; w < NW; ++w) m = fmaxf(m, wmax[w][t]);
        sx[t] = m > 0.0f ? m / 448.0f : 1.0f;
    }
    const bool dump = a.x_codes_out && tile == 0 && slot == 0;
    for (int p = tid; p < Hh; p += blockDim.x) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint32_t xx = *(const uint32_t*)(a.xin + (size_t)t * H + 2 * p);
            const uint32_t q = e4m3_pack2(bf16_to_f32((uint16_t)(xx & 0xffffu)) / sx[t],
                                          bf16_to_f32((uint16_t)(xx >> 16)) / sx[t]);
            xh[t * Hh + p] = e4m3x2_to_f16x2(q);
            if (dump) *(uint16_t*)(a.x_codes_out + (size_t)t * H + 2 * p) = (uint16_t)q;
        }
    }
    if (a.x_scale_out && tile == 0 && slot == 0 && tid < T) a.x_scale_out[tid] = sx[tid];
    __syncthreads();

    // 3. block dot products: 8 blocks of 32 codes per lane, for each routed token
    float acc[T];
#pragma unroll
    for (int j = 0; j < T; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < kGuBlocksPerWave; ++i) {
        const float scale = e8m0_to_f32(i < 4 ? sc.x >> (8 * i) : sc.y >> (8 * (i - 4)));
        const int pbase = (wv * kGuBlocksPerWave + i) * (kBlock / 2);
        const half2_t* xp[T];
#pragma unroll
        for (int j = 0; j < T; ++j) xp[j] = xh + tok[j] * Hh + pbase;
        float p[T];
#pragma unroll
        for (int j = 0; j < T; ++j) p[j] = 0.0f;
        block_dot<T>(wr[i], xp, p, ntok);
#pragma unroll
        for (int j = 0; j < T; ++j) acc[j] = fmaf(p[j], scale, acc[j]);
    }
#pragma unroll
    for (int j = 0; j < T; ++j)
        if (j < ntok) red[wv][j][lane] = acc[j];
    __syncthreads();

    // 4. sum the K slices, h = SiLU(g) * u, tile max |h| (one half-wave per token and pass)
    for (int base = 0; base < kGuHalf * ntok; base += blockDim.x) {
        const int idx = base + tid, j = idx >> 5, r = idx & 31;
        const bool act = idx < kGuHalf * ntok;
        float hv = 0.0f;
        if (act) {
            float g = 0.0f, u = 0.0f;
            for (int w = 0; w < NW; ++w) {
                g += red[w][j][r];
                u += red[w][j][kGuHalf + r];
            }
            float s = sx[0];
#pragma unroll
            for (int t = 1; t < T; ++t)
                if (tok[j] == t) s = sx[t];
            g *= s;
            u *= s;
            hv = g / (1.0f + expf(-g)) * u;
            a.h[((size_t)slot * kMaxTokens + j) * I + tile * kGuHalf + r] = hv;
        }
        const float m = wave_max(fabsf(hv), 32);
        if (act && r == 0) a.hamax[((size_t)slot * kMaxTokens + j) * (I / kGuHalf) + tile] = m;
    }
}

// ------------------------------------------------------------------------------------------------
// down GEMV + routing-weighted combine + residual
// ------------------------------------------------------------------------------------------------

struct DownArgs {
    const uint4* w2;        // repacked codes of this layer
    const uint8_t* w2s;     // repacked scales
    const SlotTable* slots;
    const float* h;         // [kMaxSlots][kMaxTokens][I]
    const float* hamax;     // [kMaxSlots][kMaxTokens][I/32]
    const uint16_t* xres;   // [T][H] residual x_l, or null
    uint16_t* xnext;        // [T][H] bf16(x_l + y), or null
    float* y;               // [T][H] or null
    int H, I;
};

template <int KSUB, int ITERS, int T, int SPW>
__global__ __launch_bounds__(768) void down_kernel(DownArgs a) {
    constexpr int R = kWave / KSUB;
    constexpr int kMaxPairs = kMaxTokens * kMaxTopK + kMaxTokens;
    extern __shared__ uint4 smem_dn[];
    half2_t* hh = (half2_t*)smem_dn;  // [pairs][I/2]
    __shared__ int pr_slot[kMaxPairs], pr_j[kMaxPairs];
    __shared__ float pr_sh[kMaxPairs], pr_coef[kMaxPairs];
    __shared__ int slot_pair0[kMaxSlots];
    __shared__ int s_npairs;
    __shared__ float red[16][T][R];
    const SlotTable* st = a.slots;
    const int n = st->n;
    const int H = a.H, I = a.I, NB = I / kBlock, Ih = I / 2, tiles = H / R;
    const int tile = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, NW = blockDim.x >> 6;

    if (tid == 0) {
        int p = 0;
        for (int s = 0; s < n; ++s) {
            slot_pair0[s] = p;
            const int nt = st->ntok[s];
            for (int j = 0; j < nt; ++j) {
                pr_slot[p] = s;
                pr_j[p] = j;
                ++p;
            }
        }
        s_npairs = p;
    }

    // 1. weight loads for this wave's slots
    uint4 wr[SPW][ITERS];
    uint32_t sb[SPW][ITERS];
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
        const int s = wv + NW * m;
        if (s < n) {
            const size_t base = (((size_t)st->expert[s] * tiles + tile) * ITERS) * kWave + lane;
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                wr[m][it] = ld_nt(a.w2 + base + (size_t)it * kWave);
                sb[m][it] = __builtin_nontemporal_load(a.w2s + base + (size_t)it * kWave);
            }
        }
    }
    __syncthreads();

    // 2. FP8 requantisation of every (slot, token) h vector: s_h = max|h| / 448
    const int npairs = s_npairs;
    if (tid < npairs) {
        const int s = pr_slot[tid], j = pr_j[tid];
        const float* am = a.hamax + ((size_t)s * kMaxTokens + j) * (I / kGuHalf);
        float m = 0.0f;
        for (int b = 0; b < I / kGuHalf; ++b) m = fmaxf(m, am[b]);
        const float sh = m > 0.0f ? m / 448.0f : 1.0f;
        pr_sh[tid] = sh;
        pr_coef[tid] = st->w[s][j] * sh;
    }
    __syncthreads();
    for (int idx = tid; idx < npairs * Ih; idx += blockDim.x) {
        const int p = idx / Ih, q = idx - p * Ih;
        const float* hp = a.h + ((size_t)pr_slot[p] * kMaxTokens + pr_j[p]) * I;
        const float2 v = *(const float2*)(hp + 2 * q);
        const float sh = pr_sh[p];
        hh[idx] = e4m3x2_to_f16x2(e4m3_pack2(v.x / sh, v.y / sh));
    }
    __syncthreads();

    // 3. down block dot products, weighted into per-token accumulators
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.0f;
    const int ks = lane % KSUB;
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
        const int s = wv + NW * m;
        if (s < n) {
            const int p0 = slot_pair0[s], nt = st->ntok[s];
            float pj[T];
#pragma unroll
            for (int j = 0; j < T; ++j) pj[j] = 0.0f;
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                const float scale = e8m0_to_f32(sb[m][it]);
                const int pbase = (it * KSUB + ks) * (kBlock / 2);
                const half2_t* xp[T];
#pragma unroll
                for (int j = 0; j < T; ++j) xp[j] = hh + (p0 + j) * Ih + pbase;
                float q[T];
#pragma unroll
                for (int j = 0; j < T; ++j) q[j] = 0.0f;
                block_dot<T>(wr[m][it], xp, q, nt);
#pragma unroll
                for (int j = 0; j < T; ++j) pj[j] = fmaf(q[j], scale, pj[j]);
            }
#pragma unroll
            for (int j = 0; j < T; ++j) {
                if (j < nt) {
                    const int tk = st->tok[s][j];
                    const float cf = pr_coef[p0 + j];
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        if (t == tk) acc[t] = fmaf(cf, pj[j], acc[t]);
                }
            }
        }
    }

    // 4. reduce over the KSUB lanes of a row, then over waves in wave order
#pragma unroll
    for (int t = 0; t < T; ++t)
        for (int off = 1; off < KSUB; off <<= 1) acc[t] += __shfl_xor(acc[t], off, 64);
    if (ks == 0) {
#pragma unroll
        for (int t = 0; t < T; ++t) red[wv][t][lane / KSUB] = acc[t];
    }
    __syncthreads();
    for (int idx = tid; idx < R * T; idx += blockDim.x) {
        const int t = idx / R, r = idx - t * R;
        float ysum = 0.0f;
        for (int w = 0; w < NW; ++w) ysum += red[w][t][r];
        const size_t o = (size_t)t * H + (size_t)tile * R + r;
        if (a.y) a.y[o] = ysum;
        if (a.xnext) a.xnext[o] = f32_to_bf16(bf16_to_f32(a.xres[o]) + ysum);
    }
}

// ------------------------------------------------------------------------------------------------
// host-side launchers (called from moe_api.cpp)
// ------------------------------------------------------------------------------------------------

static unsigned grid_for(uint64_t total, unsigned block) {
    uint64_t g = (total + block - 1) / block;
    if (g > 65536) g = 65536;
    if (g == 0) g = 1;
    return (unsigned)g;
}

hipError_t launch_repack(const Shape& sh, const void* router, const void* w13, const void* w13s, const void* w2,
                         const void* w2s, void* d_router, void* d_w13, void* d_w13s, void* d_w2, void* d_w2s,
                         hipStream_t stream) {
    const int nexp = sh.E + sh.S;
    const unsigned B = 256;
    repack_router<<<grid_for((uint64_t)sh.RT() * kRouterRows * sh.H / 8, B), B, 0, stream>>>(
        (const uint16_t*)router, (uint4*)d_router, sh.E, sh.H, sh.RT());
    repack_w13<<<grid_for((uint64_t)nexp * sh.I * sh.H / 16, B), B, 0, stream>>>((const uint4*)w13, (uint4*)d_w13,
                                                                                  nexp, sh.I, sh.H);
    repack_w13s<<<grid_for((uint64_t)nexp * 2 * sh.I * sh.H / 32 / 8, B), B, 0, stream>>>(
        (const uint8_t*)w13s, (uint2*)d_w13s, nexp, sh.I, sh.H);
    repack_w2<<<grid_for((uint64_t)nexp * sh.H * sh.I / 32, B), B, 0, stream>>>(
        (const uint4*)w2, (uint4*)d_w2, nexp, sh.H, sh.I, sh.down_ksub());
    repack_w2s<<<grid_for((uint64_t)nexp * sh.H * sh.I / 32, B), B, 0, stream>>>(
        (const uint8_t*)w2s, (uint8_t*)d_w2s, nexp, sh.H, sh.I, sh.down_ksub());
    return hipGetLastError();
}

int down_spw(int T) { return T == 1 ? 1 : T == 2 ? 2 : 3; }

int max_slots(const Shape& sh, int T) {
    const int routed = T * sh.k < sh.E ? T * sh.k : sh.E;
    return routed + sh.S;
}

template <int T>
static hipError_t launch_layer_t(const Shape& sh, const LayerPtrs& L, const RunPtrs& P, bool normalize,
                                 hipStream_t stream, hipEvent_t* ev) {
    if (ev) (void)hipEventRecord(ev[0], stream);
    RouterArgs ra{(const uint4*)L.router, P.x, P.xin, P.trace, P.partial, P.ticket, P.slots, P.ids, P.w,
                  sh.H, sh.E, sh.k, sh.S, normalize ? 1 : 0};
    router_kernel<T><<<dim3(sh.H / kRouterSlice, sh.RT()), 256, 0, stream>>>(ra);
    if (ev) (void)hipEventRecord(ev[1], stream);

    const int slots = max_slots(sh, T);
    GateUpArgs ga{(const uint4*)L.w13, (const uint2*)L.w13s, P.xin, P.slots, P.h, P.hamax, P.x_scale, P.x_codes,
                  sh.H, sh.I};
    gateup_kernel<T><<<dim3(sh.I / kGuHalf, slots), 64 * (sh.H / kGuSlice), (size_t)T * sh.H * 2, stream>>>(ga);
    if (ev) (void)hipEventRecord(ev[2], stream);

    DownArgs da{(const uint4*)L.w2, (const uint8_t*)L.w2s, P.slots, P.h, P.hamax, P.xnext ? P.x : nullptr,
                P.xnext, P.y, sh.H, sh.I};
    const int spw = down_spw(T);
    const int nw = (slots + spw - 1) / spw;
    const int pairs = T * sh.k + (sh.S ? T : 0);
    const size_t lds = (size_t)pairs * sh.I * 2;
    const int ksub = sh.down_ksub(), iters = sh.down_iters();
    const dim3 grid(sh.H / sh.down_rows());
    const unsigned block = 64 * nw;
    constexpr int S = T == 1 ? 1 : T == 2 ? 2 : 3;
    if (ksub == 2 && iters == 1) down_kernel<2, 1, T, S><<<grid, block, lds, stream>>>(da);
    else if (ksub == 4 && iters == 1) down_kernel<4, 1, T, S><<<grid, block, lds, stream>>>(da);
    else if (ksub == 4 && iters == 2) down_kernel<4, 2, T, S><<<grid, block, lds, stream>>>(da);
    else if (ksub == 4 && iters == 4) down_kernel<4, 4, T, S><<<grid, block, lds, stream>>>(da);
    else if (ksub == 4 && iters == 6) down_kernel<4, 6, T, S><<<grid, block, lds, stream>>>(da);
    else return hipErrorInvalidValue;
    if (ev) (void)hipEventRecord(ev[3], stream);
    return hipGetLastError();
}

hipError_t launch_layer(const Shape& sh, int T, const LayerPtrs& L, const RunPtrs& P, bool normalize,
                        hipStream_t stream, hipEvent_t* ev) {
    switch (T) {
        case 1: return launch_layer_t<1>(sh, L, P, normalize, stream, ev);
        case 2: return launch_layer_t<2>(sh, L, P, normalize, stream, ev);
        case 3: return launch_layer_t<3>(sh, L, P, normalize, stream, ev);
        case 4: return launch_layer_t<4>(sh, L, P, normalize, stream, ev);
        default: return hipErrorInvalidValue;
    }
}

bool down_supported(int I) {
    const int nb = I / kBlock;
    if (I % kBlock) return false;
    if (nb == 2) return true;
    return nb % 4 == 0 && (nb / 4 == 1 || nb / 4 == 2 || nb / 4 == 4 || nb / 4 == 6);
}

}  // namespace moe
