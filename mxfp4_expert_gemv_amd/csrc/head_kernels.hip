// head_kernels.hip -- FP8 LM-head GEMV with a fused per-token argmax (gfx950).
//
// The head is the 157,184 x 2,560 vocabulary projection that is read in full for every generated
// token and is quantised to FP8 at load time to halve those reads (tanhow.com, "NVIDIA 在单台 DGX
// Spark 上叠加三项优化...", section "三项优化是什么", item 2; devotd.net,
// "dgx-spark-moe-inference-optimizations", section 2).  Weights are OCP E4M3 with one fp32 scale
// per row; x stays bf16; logits are fp32; argmax takes the lowest index among equal maxima.
//
// The same kernel also runs the unquantised BF16 head (bf16_head_create), for comparison.
//
// As many workgroups as the device holds at once each walk 64-row tiles (blockIdx.x, + grid, ...),
// the next tile's first weight loads issued while the current tile finishes, and keep each token's
// best (value, lowest index) in registers; one partial per workgroup goes to the final argmax (one
// tile per workgroup, with a write-through partial and an arrival per tile, measured 81 against 67
// us for the E4M3 head).  A workgroup has H / 256 waves; wave w takes K [256 w, 256 w + 256) of the
// tile's rows on the matrix cores: v_mfma_f32_16x16x32_bf16 on four 16-row groups, A = the
// weights (E4M3 codes converted exactly to bf16 in VGPRs, or the bf16 weights themselves), B = x
// (bf16, from LDS; column n = token n, zero columns past T), fp32 accumulators.  Measured on gfx950,
// one such instruction is within 2.7 * 2^-24 * sum |terms| of the exact sum (C + 32 products), so
// the logits stay inside the any-order fp32 summation bound the argmax margin rule is built on.
// At one token 15 of the 16 B columns are zero; the instruction still beat a VALU dot product
// (v_dot2_f32_bf16) on the same registers, which needs one dot per code and token.
//
// Layout (repacked at create): [ceil(V/64) tiles][H/256 waves][U units][64 lanes][16 B], each wave-
// wide 16-byte load reading 1 KiB of contiguous HBM, in the order the blocks consume them.  Lane l,
// unit u = 4 s + r covers row 16 r + l % 16 of the tile: E4M3 (U = 16, s < 4): K 256 w + 64 s +
// 16 (l / 16) .. +16, whose two halves are the lane's A operands of MFMA blocks 2 s and 2 s + 1;
// BF16 (U = 32, s < 8): K 256 w + 32 s + 8 (l / 16) .. +8, the A operand of block s.  The B operand
// of block j for lane l is x at the same K offsets.  The last workgroup to finish reduces the
// per-tile (max, index) pairs.
//
// fp8_head_run_noalloc runs the same kernel on the caller's row-major matrix, read at the same K
// offsets, so that its logits equal the handle's bit for bit.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

namespace head {

constexpr int kWave = 64;
constexpr int kSlice = 256;  // K elements per wave: 16 units of 16 E4M3 codes, or 32 units of 8 bf16
constexpr int kNoAllocMaxVocab = 262144;  // largest vocabulary of fp8_head_run_noalloc (its scratch size)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t comp(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Row-major [V][H] -> the tile layout above (a permutation of 16-byte units; rows past V are zero,
// with scale 0).  NU 16-byte units per row: H / 16 (E4M3) or H / 8 (bf16); ssrc null: scales of 1.
__global__ void repack_head(const uint4* __restrict__ src, const float* __restrict__ ssrc, uint4* __restrict__ dst,
                            float* __restrict__ sdst, int V, int NU, int VT) {
    const int NW = NU / 16 / (ssrc ? 1 : 2);  // waves per tile (H / 256)
    const int U = NU / NW;                   // units per lane and wave
    const uint64_t total = (uint64_t)VT * NU * kWave;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(i % kWave);
        uint64_t r = i / kWave;
        const int u = (int)(r % U);
        r /= U;
        const int w = (int)(r % NW);
        const uint64_t vt = r / NW;
        const uint64_t row = vt * kWave + 16 * (u % 4) + (lane & 15);
        // first unit of the wave's K slice, plus the unit's step within it (4 units per 64 K of
        // E4M3, 4 per 32 K of bf16), plus the lane's quarter
        const int unit = w * U + 4 * (u / 4) + (lane >> 4);
        dst[i] = row < (uint64_t)V ? src[row * NU + unit] : make_uint4(0, 0, 0, 0);
        if (u < 4 && lane < 16 && w == 0) sdst[row] = row < (uint64_t)V ? (ssrc ? ssrc[row] : 1.0f) : 0.0f;
    }
}

struct HeadArgs {
    const uint4* w;       // repacked E4M3
    const float* scale;   // [VT*64], zero past V
    const uint16_t* x;    // [T][H] bf16
    float* logits;        // [T][V] or null
    int32_t* argmax;      // [T]
    float* pval;          // [grid][T] per-workgroup maxima (room for [VT][T])
    int32_t* pidx;        // [grid][T]
    unsigned* ticket;
    const int32_t* draft;  // [T-1] drafted tokens of positions 1 .. T-1, or null
    int32_t* accept;       // [1] accepted drafts (with draft)
    int V, H;
    int VT;                // 64-row tiles (the grid is smaller: each workgroup walks several)
};

__device__ __forceinline__ void better(float& bv, int& bi, float ov, int oi) {
    if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
    }
}

// One tile's end: red[w][t][r] holds wave w's partial sum of row r of tile vt for token t.  Wave
// t % NW sums the waves, scales, writes the logits and folds the tile's (max, lowest index) into
// token t's running best (bv[t], bi[t]), the same in every lane of the wave.
template <int T>
__device__ void tile_best(const HeadArgs& a, const float (*red)[T][kWave], int vt, float (&bv)[T], int (&bi)[T]) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, NW = blockDim.x >> 6;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if (t % NW != wv) continue;  // uniform per wave
        float s = 0.0f;
        for (int w = 0; w < NW; ++w) s += red[w][t][lane];
        const int row = vt * kWave + lane;
        float v = -INFINITY;
        int idx = 0x7fffffff;
        if (row < a.V) {
            v = s * a.scale[row];
            idx = row;
            if (a.logits) a.logits[(size_t)t * a.V + row] = v;
        }
        for (int off = 32; off > 0; off >>= 1) better(v, idx, __shfl_xor(v, off, 64), __shfl_xor(idx, off, 64));
        better(bv[t], bi[t], v, idx);
    }
}

// The end of the head kernel: each token's best over this workgroup's tiles is its partial; the
// last workgroup to arrive reduces the partials of all workgroups (and the verify acceptance).
template <int T>
__device__ void head_finish(const HeadArgs& a, const float (&bv)[T], const int (&bi)[T], int* is_last) {
    const int G = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, NW = blockDim.x >> 6;
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if (t % NW == wv && lane == 0) {  // write-through: the last workgroup reads them without any cache flush
            __hip_atomic_store(a.pval + (size_t)blockIdx.x * T + t, bv[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.pidx + (size_t)blockIdx.x * T + t, bi[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // the last workgroup to arrive reduces the partials.  Ordering rests on the ISA, not on
    // release/acquire (its L2 write-back in every workgroup costs the head about 15 us): the
    // partials are agent-scope atomic stores, written through to the device-coherent level,
    // vmcnt(0) waits for the memory's acknowledgement before the arrival, and the last workgroup
    // reads them with agent-scope atomic loads, which do not hit in the non-coherent L2.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0)
        *is_last = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(G - 1);
    __syncthreads();
    if (!*is_last) return;
    __shared__ int32_t am_s[T];
    for (int t = wv; t < T; t += NW) {
        float v = -INFINITY;
        int idx = 0x7fffffff;
        for (int i = lane; i < G; i += kWave)
            better(v, idx, __hip_atomic_load(a.pval + (size_t)i * T + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                   __hip_atomic_load(a.pidx + (size_t)i * T + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        for (int off = 32; off > 0; off >>= 1) better(v, idx, __shfl_xor(v, off, 64), __shfl_xor(idx, off, 64));
        if (lane == 0) {
            a.argmax[t] = idx;
            am_s[t] = idx;
        }
    }
    if (a.draft) {
        // greedy acceptance of a speculative verify step: the drafts are kept while each equals the
        // target's token of the position before it
        __syncthreads();
        if (tid == 0) {
            int n = 0;
            while (n < T - 1 && am_s[n] == a.draft[n]) ++n;
            *a.accept = n;
        }
    }
    if (tid == 0) *a.ticket = 0u;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 8 E4M3 codes (two dwords) -> the bf16 A operand of one MFMA block (exact).
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint32_t d0, uint32_t d1) {
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, 1.0f, false);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, 1.0f, true);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, 1.0f, false);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, 1.0f, true);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Register use: the wave's weights stream through a ring of RS steps (4 units each, one per 16-row
// group): the loads of step s + RS are issued as soon as step s has been consumed, so a lane holds
// 4 RS units instead of all of its 16 (E4M3) or 32 (bf16).  Occupancy: E4M3 at most 80 VGPRs (6
// waves per SIMD), bf16 at most 64 (8 waves), so that two 10-wave workgroups (3, 3, 2, 2 waves on
// the four SIMDs) always share a compute unit; all 16 units in registers (96 VGPRs, 5 waves) made
// the head a third slower.  Measured on the 157,184 x 2,560 head: E4M3 with 2 steps (77-79 VGPRs)
// and bf16 with 1 step (59-61) were the fastest of 1-4 steps at 6 and 8 waves.  The row-major form
// takes 1 step: with 2 its row addresses spilled to scratch.
template <bool FP8, bool RM>
constexpr int head_ring_steps() { return FP8 && !RM ? 2 : 1; }
template <int T, bool FP8, bool RM = false>
__global__ __launch_bounds__(640) __attribute__((amdgpu_waves_per_eu(6))) void head_mfma(HeadArgs a) {
    constexpr int U = FP8 ? 16 : 32;  // units per lane
    constexpr int S = U / 4;          // steps
    constexpr int RS = head_ring_steps<FP8, RM>();
    static_assert(S % RS == 0, "a step keeps its ring slot from tile to tile");
    extern __shared__ uint32_t xs[];  // [T][H/2] bf16 pairs
    __shared__ float red[10][T][kWave];
    __shared__ int is_last;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, NW = blockDim.x >> 6;
    const int H = a.H, Hh = H / 2, VT = a.VT, G = gridDim.x;

    uint4 wr[4 * RS];
    // step st of tile vt: unit 4 st + r of the lane (16-row group r) into ring slot st % RS.  Row-
    // major: a 32-bit unit index (the caller's matrix is at most MOE_NOALLOC_MAX_VOCAB x 2560 bytes).
    auto issue = [&](int vt, int st) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (RM) {
                static_assert(FP8, "row-major weights are E4M3");
                const uint32_t row = (uint32_t)min(vt * kWave + 16 * r + (lane & 15), a.V - 1);
                wr[(st % RS) * 4 + r] = ld_nt(a.w + (row * (uint32_t)(H / 16) + wv * U + (lane >> 4) + 4 * st));
            } else {
                wr[(st % RS) * 4 + r] = ld_nt(a.w + ((((size_t)vt * NW + wv) * U + 4 * st + r) * kWave + lane));
            }
        }
    };
    int vt = blockIdx.x;  // this workgroup's tiles: blockIdx.x, + G, + 2 G, ... (G <= VT)
#pragma unroll
    for (int st = 0; st < RS; ++st) issue(vt, st);
    for (int i = tid; i < T * Hh; i += blockDim.x) xs[i] = ((const uint32_t*)a.x)[i];
    __syncthreads();

    const int n = lane & 15, g = lane >> 4;
    const bool on = n < T;
    const uint16_t* xrow = (const uint16_t*)xs + (on ? n : 0) * H + wv * 256;
    float bv[T];  // token t's best over the workgroup's tiles (held by wave t % NW)
    int bi[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        bv[t] = -INFINITY;
        bi[t] = 0x7fffffff;
    }
    for (; vt < VT; vt += G) {
        const int nvt = vt + G;
        f32x4_t acc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < S; ++st) {
            // E4M3: the step's units hold blocks 2 st and 2 st + 1 (their low and high halves); bf16:
            // block st
#pragma unroll
            for (int h = 0; h < (FP8 ? 2 : 1); ++h) {
                const int kofs = FP8 ? 64 * st + 16 * g + 8 * h : 32 * st + 8 * g;
                uint4 xb = make_uint4(0, 0, 0, 0);
                if (on) xb = *(const uint4*)(xrow + kofs);
                const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xb);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint4& q = wr[(st % RS) * 4 + r];
                    bf16x8_t w;
                    if constexpr (FP8)
                        w = h ? e4m3x8_to_bf16x8(q.z, q.w) : e4m3x8_to_bf16x8(q.x, q.y);
                    else
                        w = __builtin_bit_cast(bf16x8_t, q);
                    acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, b, acc[r], 0, 0, 0);
                }
            }
            // refill the slot: a later step of this tile, or the first steps of the next one
            if (st + RS < S)
                issue(vt, st + RS);
            else if (nvt < VT)
                issue(nvt, st + RS - S);
        }
        // lane l holds rows 16 r + 4 (l / 16) + i of the tile for token l % 16
        if (on) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[wv][n][16 * r + 4 * g + i] = acc[r][i];
        }
        __syncthreads();
        tile_best<T>(a, red, vt, bv, bi);
        __syncthreads();  // red is rewritten by the next tile
    }
    head_finish<T>(a, bv, bi, &is_last);
}

// Per-row FP8 quantisation of the head at load time (the step the pages put before the FP8 head):
// s_r = fl32(max_c |W[r][c]| / 448), 1 for an all-zero row, and code[r][c] = E4M3 round-to-nearest-
// even of fl32(W[r][c] / s_r) (both divisions correctly rounded; |W / s| <= 448 up to the rounding
// of s, inside the E4M3 range).  One wave per row: lane l holds the 8-element chunks l, l + 64, ...
// of the row (H / 8 <= 320 chunks, so at most 5 per lane), one wave-wide maximum, then the codes.
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_rows(const void* __restrict__ w, int V, int H,
                                                     uint8_t* __restrict__ codes, float* __restrict__ scales) {
    constexpr int kChunks = 5;
    const int lane = threadIdx.x & 63, row = blockIdx.x * 4 + (threadIdx.x >> 6), NC = H / 8;
    if (row >= V) return;  // the whole wave
    float v[kChunks][8];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
        const int c = lane + 64 * j;
        if (c < NC) {
            if constexpr (BF16) {
                const uint4 u = ((const uint4*)w)[(size_t)row * NC + c];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[j][2 * q] = __uint_as_float(comp(u, q) << 16);
                    v[j][2 * q + 1] = __uint_as_float(comp(u, q) & 0xffff0000u);
                }
            } else {
                const float4 a = ((const float4*)w)[((size_t)row * NC + c) * 2];
                const float4 b = ((const float4*)w)[((size_t)row * NC + c) * 2 + 1];
                v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
                v[j][4] = b.x; v[j][5] = b.y; v[j][6] = b.z; v[j][7] = b.w;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
        }
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const float s = m > 0.0f ? m / 448.0f : 1.0f;
    if (lane == 0) scales[row] = s;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
        const int c = lane + 64 * j;
        if (c < NC) {
            uint32_t d[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float a = v[j][2 * q] / s, b = v[j][2 * q + 1] / s;
                d[q] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
                // the hardware conversion writes 0xFF for every NaN; keep the NaN's sign (S.1111.111)
                if (__builtin_isnan(a)) d[q] = (d[q] & 0xff00u) | ((__float_as_uint(a) >> 24) & 0x80u) | 0x7fu;
                if (__builtin_isnan(b)) d[q] = (d[q] & 0x00ffu) | ((((__float_as_uint(b) >> 24) & 0x80u) | 0x7fu) << 8);
            }
            ((uint2*)codes)[(size_t)row * NC + c] = make_uint2(d[0] | (d[1] << 16), d[2] | (d[3] << 16));
        }
    }
}

hipError_t launch_quantize_rows(const void* w, bool bf16, int V, int H, void* codes, float* scales,
                                hipStream_t stream) {
    const unsigned grid = (unsigned)((V + 3) / 4);
    if (bf16)
        quantize_rows<true><<<grid, 256, 0, stream>>>(w, V, H, (uint8_t*)codes, scales);
    else
        quantize_rows<false><<<grid, 256, 0, stream>>>(w, V, H, (uint8_t*)codes, scales);
    return hipGetLastError();
}

// w: E4M3 [V][H] with scales s (fp8), or bf16 [V][H] (s ignored, scales of 1)
hipError_t launch_repack_head(const void* w, const void* s, void* dw, void* ds, int V, int H, bool fp8,
                              hipStream_t stream) {
    const int VT = (V + kWave - 1) / kWave, NU = fp8 ? H / 16 : H / 8;
    uint64_t total = (uint64_t)VT * NU * kWave;
    uint64_t g = (total + 255) / 256;
    if (g > 65536) g = 65536;
    repack_head<<<(unsigned)g, 256, 0, stream>>>((const uint4*)w, fp8 ? (const float*)s : nullptr, (uint4*)dw,
                                                 (float*)ds, V, NU, VT);
    return hipGetLastError();
}

// The grid: at most as many workgroups as the device holds at once (each walks tiles blockIdx.x,
// + grid, ...), and no more than the number of rounds those need: with the tiles spread evenly, the
// last round keeps nearly every workgroup busy (157,184 rows: 492 workgroups of 5 tiles, not 512 of
// which 104 idle through the fifth round).
template <int T, bool FP8, bool RM>
static hipError_t launch_head_tt(const HeadArgs& a, hipStream_t stream) {
    const unsigned block = kWave * (a.H / kSlice);
    const size_t lds = (size_t)T * a.H * 2;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, head_mfma<T, FP8, RM>, block, lds);
    if (e != hipSuccess) return e;
    const int cap = std::max(per_cu, 1) * std::max(cus, 1), rounds = (a.VT + cap - 1) / cap;
    const int grid = (a.VT + rounds - 1) / rounds;
    head_mfma<T, FP8, RM><<<grid, block, lds, stream>>>(a);
    return hipGetLastError();
}

template <bool FP8, bool RM = false>
static hipError_t launch_head_t(const HeadArgs& a, int T, hipStream_t stream) {
    switch (T) {
        case 1: return launch_head_tt<1, FP8, RM>(a, stream);
        case 2: return launch_head_tt<2, FP8, RM>(a, stream);
        case 3: return launch_head_tt<3, FP8, RM>(a, stream);
        case 4: return launch_head_tt<4, FP8, RM>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_head(const void* w, const float* scale, const uint16_t* x, int T, float* logits, int32_t* argmax,
                       float* pval, int32_t* pidx, unsigned* ticket, const int32_t* draft, int32_t* accept, int V,
                       int H, bool fp8, hipStream_t stream) {
    const int VT = (V + kWave - 1) / kWave;
    HeadArgs a{(const uint4*)w, scale, x, logits, argmax, pval, pidx, ticket, draft, accept, V, H, VT};
    return fp8 ? launch_head_t<true>(a, T, stream) : launch_head_t<false>(a, T, stream);
}

// ------------------------------------------------------------------------------------------------
// The head without a handle, for callers that cannot allocate: its scratch (the arrival counter and
// the per-workgroup maxima of the argmax reduction) is this fixed device array, one copy per GPU that
// the library runs on, held until the process ends.  Host code never passes the array's name to a
// kernel (in host code it is a stand-in, not a device address); it passes the address that
// hipGetSymbolAddress returns for the current device.
// ------------------------------------------------------------------------------------------------

constexpr int kNoAllocMaxTiles = kNoAllocMaxVocab / kWave;
constexpr size_t kScratchTicket = 0;                                                 // unsigned, zero between calls
constexpr size_t kScratchVal = 256;                                                  // float [tiles][4]
constexpr size_t kScratchIdx = kScratchVal + (size_t)kNoAllocMaxTiles * 4 * 4;       // int32 [tiles][4]
constexpr size_t kScratchBytes = kScratchIdx + (size_t)kNoAllocMaxTiles * 4 * 4;     // 131,328 bytes

static __device__ __align__(256) uint8_t scratch[kScratchBytes];  // zero when the library is loaded

constexpr int kMaxDevices = 64;
static void* g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of the scratch array on the current device (looked up once per device).
hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

// fp8_head_run's kernel on row-major E4M3 weights [V][H] and scales [V], with the scratch above
// (V <= kNoAllocMaxVocab, checked by the caller).
hipError_t launch_head_rowmajor(const void* w, const float* scale, const uint16_t* x, int T, float* logits,
                                int32_t* argmax, void* scratch_dev, int V, int H, hipStream_t stream) {
    const int VT = (V + kWave - 1) / kWave;
    uint8_t* sp = (uint8_t*)scratch_dev;
    HeadArgs a{(const uint4*)w, scale, x, logits, argmax, (float*)(sp + kScratchVal), (int32_t*)(sp + kScratchIdx),
               (unsigned*)(sp + kScratchTicket), nullptr, nullptr, V, H, VT};
    return launch_head_t<true, true>(a, T, stream);
}

}  // namespace head

namespace probe {

// Reads n16 16-byte units with the weight kernels' load (16 bytes per lane, non-temporal), several
// independent loads in flight per lane, and folds them into one word per workgroup so that the
// loads are kept.  The practical HBM read ceiling of this access pattern.
__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ src, uint64_t n16, uint32_t* out) {
    constexpr int kUnroll = 8;
    uint32_t acc = 0;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        uint4 v[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) v[j] = head::ld_nt(src + i + j * stride);
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = head::ld_nt(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int t = 0; t < (int)blockDim.x; ++t) r ^= red[t];
        out[blockIdx.x] = r;
    }
}

hipError_t launch_stream_read(const void* src, uint64_t bytes, uint32_t* out, int grid, hipStream_t stream) {
    stream_read<<<grid, 256, 0, stream>>>((const uint4*)src, bytes / 16, out);
    return hipGetLastError();
}

}  // namespace probe
