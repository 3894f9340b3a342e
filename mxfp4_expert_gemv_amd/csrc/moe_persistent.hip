// moe_persistent.hip -- the whole decode stack (every layer, every step) in one persistent,
// cooperatively launched kernel for gfx950.
//
// One workgroup of 512 threads per compute unit stays resident for the whole pass.  Per layer the
// workgroups exchange data four times through small stamped buffers instead of kernel boundaries:
//
//   round X  the layer input x_l: every workgroup owns a few hidden rows, publishes bf16(x + y) for
//            them at the end of the previous layer and reads the whole vector;
//   round R  router logits and the shared expert's h: every workgroup owns E/N router rows and I/N
//            of the shared expert's SwiGLU outputs (neither depends on routing, so their weights
//            are loaded before x arrives); every workgroup then takes the top-k of every token
//            itself (one wave per token) and builds the same list of distinct routed experts;
//   round H  the routed experts' h: the workgroups are split into one group per routed expert; a
//            group streams that expert's MXFP4 gate/up rows (I/group outputs per workgroup) and
//            its down rows (H/group rows per workgroup), issued together right after the top-k;
//            the group's members exchange h, requantise it to FP8 and finish their down rows;
//   round D  the routed down outputs: each workgroup gathers, for its own hidden rows, the k
//            routed terms of every token and adds them in rank order to the shared expert's term
//            (computed locally), then publishes the next layer's input (round X).
//
// Every exchanged word is 64 bits: the payload in the low half and a stamp that is unique to the
// (pass, layer) in the high half, written with device-scope stores and polled with device-scope
// loads, so a reader never needs a fence or a separate flag.  Every workgroup publishes in every
// round, so no workgroup can run more than one round ahead of another; buffers alternate by layer
// parity.  Every wait is bounded in wall-clock time: on expiry the workgroup raises a device-wide
// abort flag that every other wait checks, and all workgroups leave the kernel.
//
// What is computed follows the MoE decode step described on the pages (tanhow.com, "NVIDIA 在单台
// DGX Spark 上叠加三项优化..." sections "Ling 3.0 是什么" (8 of 512 routed experts + 1 shared) and
// "三项优化是什么" items 1 and 3 (width-768 MXFP4 experts; a 4-position verify touching up to 32
// experts); devotd.net "dgx-spark-moe-inference-optimizations" section 2 (MXFP4 = blocked 4-bit
// float, 4-bit weights with 8-bit activations)).  Weights stay in their canonical row-major layout:
// the lanes of a wave read consecutive 16-byte MX blocks of a row, so loads are contiguous.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "moe_device.h"
#include "moe_launch.h"
#include "moe_persistent.h"

// Optional per-phase timestamps of a profiling build (empty otherwise).
#ifndef PK_MARK
#define PK_MARK(i)
#endif

namespace moe {
namespace pk {

constexpr int NTH = 512;           // threads per workgroup
constexpr int NWV = NTH / kWave;   // waves per workgroup
constexpr int RU = 5;              // router row: 16-byte units per lane (H / 8 <= 5 * 64)
constexpr int GJ = 3;              // gate/up unit: MX blocks per lane (2 * H / 32 <= 3 * 64)
constexpr int DG = 2;              // gate/up units per prefetch buffer (two buffers in flight)

// control words
constexpr int C_EPOCH = 0, C_ARRIVE = 1, C_ABORT = 2, C_CODE = 3, C_LAYER = 4, C_WG = 5;

// Every device-memory access below goes through global-address-space pointers, so it compiles to
// global_* instructions, which count only against vmcnt.  (Generic pointers, such as those read
// from the layer table, would give flat_* instructions, which also count against lgkmcnt: every
// LDS wait and workgroup barrier would then wait for all weight loads in flight.)
#define GLOBAL __attribute__((address_space(1)))
template <typename U>
__device__ __forceinline__ GLOBAL U* gp(U* p) {
    return (GLOBAL U*)p;
}
template <typename U>
__device__ __forceinline__ const GLOBAL U* gp(const U* p) {
    return (const GLOBAL U*)p;
}

__device__ __forceinline__ uint4 ldg_nt(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load((const GLOBAL u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ldg_nt_u8(const uint8_t* p) { return __builtin_nontemporal_load(gp(p)); }

__device__ __forceinline__ uint64_t aload64(const uint64_t* p) {
    return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t aload32(const uint32_t* p) {
    return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void astore64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void astore32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t word(float v, uint32_t stamp) {
    return ((uint64_t)stamp << 32) | __float_as_uint(v);
}
__device__ __forceinline__ float payload(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Stamp of layer l in pass `epoch`: never 0 (cleared buffers), different for consecutive layers.
__device__ __forceinline__ uint32_t stamp_of(uint32_t epoch, int L, int l) {
    return 1u + (uint32_t)(((uint64_t)epoch * (uint64_t)L + (uint64_t)l) % 0xFFFFFFFFull);
}

struct Wait {
    uint32_t* ctl;
    long long timeout;  // wall-clock ticks allowed per wait
    int code;           // which round (for the error report)
    int layer;
};

// Marks the pass as failed (first failure wins the report) and raises the abort flag.
__device__ void raise_abort(const Wait& w) {
    uint32_t expected = 0u;
    if (__hip_atomic_compare_exchange_strong(gp(w.ctl + C_CODE), &expected, (uint32_t)w.code, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        astore32(w.ctl + C_LAYER, (uint32_t)w.layer);
        astore32(w.ctl + C_WG, blockIdx.x);
    }
    astore32(w.ctl + C_ABORT, 1u);
}

// Words src[i0 + m * NTH] (m < M, index < n) of this thread: first loads (issued together).
template <int M>
__device__ __forceinline__ void poll_issue(const uint64_t* src, int i0, int n, uint64_t (&v)[M]) {
#pragma unroll
    for (int m = 0; m < M; ++m) v[m] = aload64(src + min(i0 + m * NTH, n - 1));
}

// Reloads the words whose stamp is not `stamp` until all carry it.  Returns false on time-out or
// when another workgroup raised the abort flag.
template <int M>
__device__ bool poll_wait(const uint64_t* src, int i0, int n, uint32_t stamp, uint64_t (&v)[M], const Wait& w) {
    const long long t0 = wall_clock64();
    for (int it = 0;; ++it) {
        bool ok = true;
#pragma unroll
        for (int m = 0; m < M; ++m) ok &= (i0 + m * NTH >= n) || (uint32_t)(v[m] >> 32) == stamp;
        if (ok) return true;
        if ((it & 7) == 7) {
            if (aload32(w.ctl + C_ABORT) != 0u) return false;
            if (wall_clock64() - t0 > w.timeout) {
                raise_abort(w);
                return false;
            }
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int i = i0 + m * NTH;
            if (i < n && (uint32_t)(v[m] >> 32) != stamp) v[m] = aload64(src + i);
        }
    }
}

// ------------------------------------------------------------------------------------------------
// work pieces
// ------------------------------------------------------------------------------------------------

// One router row (5 KiB for H = 2560): lane loads 16-byte units lane, lane + 64, ...
__device__ __forceinline__ void router_load(const uint16_t* router, int e, int H, uint4 (&w)[RU], int lane) {
    const int NU = H / 8;
    const uint4* p = (const uint4*)(router + (size_t)e * H);
#pragma unroll
    for (int j = 0; j < RU; ++j) w[j] = ldg_nt(p + min(lane + 64 * j, NU - 1));
}

template <int T>
__device__ __forceinline__ void router_dot(const uint4 (&w)[RU], int H, const uint16_t* xn, float (&acc)[T],
                                           int lane) {
    const int NU = H / 8;
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int j = 0; j < RU; ++j) {
        const int u = lane + 64 * j;
        if (u < NU) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const uint4 xv = *(const uint4*)(xn + t * H + u * 8);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t d = comp(w[j], q), xx = comp(xv, q);
                    acc[t] = fmaf(__uint_as_float(d << 16), __uint_as_float(xx << 16), acc[t]);
                    acc[t] = fmaf(__uint_as_float(d & 0xffff0000u), __uint_as_float(xx & 0xffff0000u), acc[t]);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = sum64(acc[t]);
}

// One gate/up unit: SwiGLU output i of expert e = gate row i and up row I + i over all H.  The
// wave's lanes cover the 2 * H/32 MX blocks of the two rows in order (gate blocks, then up).
struct GuUnit {
    uint4 w[GJ];
    uint32_t sc[GJ];  // scale byte of each block (kept apart: combining them would wait for the loads)
};

__device__ __forceinline__ void gu_load(const uint4* w13, const uint8_t* w13s, int e, int i, int I, int NB,
                                        GuUnit& u, int lane) {
    const size_t r0 = (size_t)e * 2 * I;
#pragma unroll
    for (int j = 0; j < GJ; ++j) {
        const int f = min(lane + 64 * j, 2 * NB - 1);
        const int sel = f >= NB ? 1 : 0;
        const int blk = f - sel * NB;
        const size_t row = r0 + (size_t)(sel ? I + i : i);
        u.w[j] = ldg_nt(w13 + row * NB + blk);
        u.sc[j] = ldg_nt_u8(w13s + row * NB + blk);
    }
}

// Gate and up sums (without the activation scale) of the nt tokens tok[q]; every lane gets them.
template <int T>
__device__ __forceinline__ void gu_dot(const GuUnit& u, int NB, const half2_t* xh, int Hh, const int (&tok)[T],
                                       int nt, float (&g)[T], float (&up)[T], int lane) {
#pragma unroll
    for (int q = 0; q < T; ++q) g[q] = up[q] = 0.0f;
#pragma unroll
    for (int j = 0; j < GJ; ++j) {
        const int f = lane + 64 * j;
        if (f < 2 * NB) {
            const bool is_up = f >= NB;
            const int blk = is_up ? f - NB : f;
            const float scale = e8m0_to_f32(u.sc[j]);
            const half2_t* xp[T];
#pragma unroll
            for (int q = 0; q < T; ++q) xp[q] = xh + tok[q] * Hh + blk * (kBlock / 2);
            float p[T];
#pragma unroll
            for (int q = 0; q < T; ++q) p[q] = 0.0f;
            block_dot<T>(u.w[j], xp, p, nt);
#pragma unroll
            for (int q = 0; q < T; ++q) {
                if (is_up) up[q] = fmaf(p[q], scale, up[q]);
                else g[q] = fmaf(p[q], scale, g[q]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < T; ++q) {
        if (q < nt) {
            g[q] = sum64(g[q]);
            up[q] = sum64(up[q]);
        }
    }
}

__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// One down pass: 64/KSUB consecutive rows of one expert, KSUB lanes per row, ITERS MX blocks per
// lane (block it * KSUB + lane % KSUB of the row).
template <int ITERS>
struct DnPass {
    uint4 w[ITERS];
    uint32_t sc[ITERS];
};

template <int KSUB, int ITERS>
__device__ __forceinline__ void dn_load(const uint4* w2, const uint8_t* w2s, int e, int row, int H, int NI,
                                        DnPass<ITERS>& d, int lane) {
    const int ks = lane % KSUB;
    const size_t r = (size_t)e * H + row;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const size_t b = r * NI + it * KSUB + ks;
        d.w[it] = ldg_nt(w2 + b);
        d.sc[it] = ldg_nt_u8(w2s + b);
    }
}

// Row sums of the pass for the nt FP8 h vectors hq + q * Ih (scaled by sh[q]); reduced over the
// KSUB lanes of the row, valid in lane % KSUB == 0.
template <int KSUB, int ITERS, int T>
__device__ __forceinline__ void dn_dot(const DnPass<ITERS>& d, const half2_t* hq, int Ih, int nt, float (&out)[T],
                                       int lane) {
    const int ks = lane % KSUB;
#pragma unroll
    for (int q = 0; q < T; ++q) out[q] = 0.0f;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const float scale = e8m0_to_f32(d.sc[it]);
        const half2_t* xp[T];
#pragma unroll
        for (int q = 0; q < T; ++q) xp[q] = hq + q * Ih + (it * KSUB + ks) * (kBlock / 2);
        float p[T];
#pragma unroll
        for (int q = 0; q < T; ++q) p[q] = 0.0f;
        block_dot<T>(d.w[it], xp, p, nt);
#pragma unroll
        for (int q = 0; q < T; ++q) out[q] = fmaf(p[q], scale, out[q]);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < T; ++q) out[q] = sum_ksub<KSUB>(out[q]);
}

// FP8 requantisation of nv vectors of I fp32 values v (value i0 + m * NTH of the concatenated
// vectors, held by this thread): s = max|h| / 448 (1 when h = 0) per vector (into scale[], LDS, by the
// first nv threads), the exact f16 values of the codes into out[vec][I] (LDS, as _Float16).  I is
// a multiple of 64, so each 64-word chunk belongs to one vector.  cmax: LDS scratch of nv * I / 64
// floats.  One barrier inside; the caller synchronises before reading out or scale.
template <int M>
__device__ void requant(const float (&v)[M], int i0, int nv, int I, float* scale, _Float16* out, float* cmax) {
    const int lane = i0 & 63, n = nv * I, CH = I / 64;  // CH <= 16
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int i = i0 + m * NTH;  // uniform chunk per wave: i / 64 is the same for all lanes
        if (i - lane < n) {
            const float mx = max64(fabsf(v[m]));
            if (lane == 0) cmax[i / 64] = mx;
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int i = i0 + m * NTH;
        if (i - lane < n) {  // uniform per wave
            const int vec = (unsigned)i / (unsigned)I;
            float cm = lane < CH ? cmax[vec * CH + lane] : 0.0f;
            cm = max16(cm);
            const float mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cm)));
            const float s = mx > 0.0f ? mx / 448.0f : 1.0f;
            if (lane == 0 && (unsigned)(i - lane) % (unsigned)I == 0u) scale[vec] = s;
            out[i] = e4m3x2_to_f16x2(e4m3_pack2(v[m] / s, 0.0f)).x;
        }
    }
}

// Top-k of every token from the logits lg[T][E] (LDS): one wave per token, each lane sorts its 8
// keys (experts lane + 64j), k rounds take the wave-wide maximum of the lanes' heads and the
// winning lane pops its head; lane r keeps the winner of round r, so the softmax over the selected
// logits runs across lanes 0..k-1.  Then the list of distinct routed experts in order of first
// appearance (token, then rank).  ids/wts/st: LDS.
template <int T>
__device__ void route_lds(const float* lg, int E, int k, SlotTable* st, int* ids, float* wts, int tid) {
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (wv < T) {
        const int t = wv;
        uint64_t key[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = lane + 64 * j;
            key[j] = e < E ? topk_key(lg[t * E + min(e, E - 1)], e) : 0ull;
        }
        cx_desc(key[0], key[1]); cx_desc(key[2], key[3]); cx_desc(key[4], key[5]); cx_desc(key[6], key[7]);
        cx_desc(key[0], key[2]); cx_desc(key[1], key[3]); cx_desc(key[4], key[6]); cx_desc(key[5], key[7]);
        cx_desc(key[1], key[2]); cx_desc(key[5], key[6]);
        cx_desc(key[0], key[4]); cx_desc(key[1], key[5]); cx_desc(key[2], key[6]); cx_desc(key[3], key[7]);
        cx_desc(key[2], key[4]); cx_desc(key[3], key[5]);
        cx_desc(key[1], key[2]); cx_desc(key[3], key[4]); cx_desc(key[5], key[6]);
        uint64_t mine = 0ull;
        for (int r = 0; r < k; ++r) {
            uint64_t best = key[0];
            best = max64u(best, xchg<0>(best));
            best = max64u(best, xchg<1>(best));
            best = max64u(best, xchg<2>(best));
            best = max64u(best, xchg<3>(best));
            best = max64u(best, xchg<4>(best));
            best = max64u(best, xchg<5>(best));
            const bool win = key[0] == best;  // keys are unique: exactly one lane pops
#pragma unroll
            for (int j = 0; j < 7; ++j) key[j] = win ? key[j + 1] : key[j];
            key[7] = win ? 0ull : key[7];
            mine = lane == r ? best : mine;
        }
        const uint32_t o = (uint32_t)(mine >> 32);
        const float lv = __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
        const float l0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(lv)));  // the maximum
        const float z = lane < k ? expf(lv - l0) : 0.0f;
        float zs = z + xchg<0>(z);
        zs += xchg<1>(zs);
        zs += xchg<2>(zs);  // lanes 0..7 hold the sum over lanes 0..7 (k <= 8)
        if (lane < k) {
            ids[t * k + lane] = (int)(0xffffffffu - (uint32_t)mine);
            wts[t * k + lane] = z / zs;
        }
    }
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
        for (int q = 0; q < np; ++q) {
            const bool same = ids[q] == e;
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

// ------------------------------------------------------------------------------------------------
// the kernel
// ------------------------------------------------------------------------------------------------

// words per thread of each polled round (largest shapes: H 2560, E 512, I 768)
template <int T>
struct Sizes {
    static constexpr int MX = (T * 1280 + NTH - 1) / NTH;           // x: T * H/2 words
    static constexpr int ML = (T * 512 + NTH - 1) / NTH;            // logits: T * E words
    static constexpr int MS = (T * 768 + NTH - 1) / NTH;            // shared h: T * I words
    static constexpr int MH = (kMaxTokens * 768 + NTH - 1) / NTH;   // routed h: ntok * I words
    static constexpr int MG = 2;                                    // gathered d: per batch
    static constexpr int DPM = 2;                                   // down passes prefetched per wave
};

template <int T, int KSUB, int ITERS>
__global__ __launch_bounds__(NTH) void stack_kernel(StackArgs a) {
    using Z = Sizes<T>;
    constexpr int UPW = kWave / KSUB;  // rows per down pass
    extern __shared__ uint4 smem[];
    __shared__ SlotTable st;
    __shared__ int ids[T * kMaxTopK];
    __shared__ float wts[T * kMaxTopK];
    __shared__ int qs[T * kMaxTopK], qj[T * kMaxTopK];  // (token, rank) -> slot, position in slot
    __shared__ float sx[T], shs[T], rhs[kMaxTokens];
    __shared__ double redd[NWV * T];
    __shared__ float redf[NWV * T];
    __shared__ uint32_t s_epoch;
    __shared__ int s_grp[2];  // own slot, its first workgroup

    if (threadIdx.x == 0) {
        const uint32_t ep = aload32(a.ctl + C_EPOCH);
        const uint32_t ab = aload32(a.ctl + C_ABORT);
        s_epoch = ab ? 0xFFFFFFFFu : ep;  // a raised abort flag makes every later pass exit at once
        if (!ab) __hip_atomic_fetch_add(gp(a.ctl + C_ARRIVE), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const uint32_t epoch = s_epoch;
    if (epoch == 0xFFFFFFFFu) return;
    const int L = a.L;
    Wait w{a.ctl, a.timeout, 0, 0};
    // fixed per-workgroup ranges (32-bit arithmetic: every product stays below 2^31)
    __shared__ int s_rng[6];
    if (threadIdx.x == 0) {
        const unsigned c = blockIdx.x, N = gridDim.x;
        s_rng[0] = (int)(c * (unsigned)a.E / N);                          // router rows [0], [1]
        s_rng[1] = (int)((c + 1) * (unsigned)a.E / N);
        s_rng[2] = a.S ? (int)(c * (unsigned)a.I / N) : 0;                // shared SwiGLU outputs [2], [3]
        s_rng[3] = a.S ? (int)((c + 1) * (unsigned)a.I / N) : 0;
        s_rng[4] = 2 * (int)(c * (unsigned)(a.H / 2) / N);                // own hidden rows [4], [5]
        s_rng[5] = 2 * (int)((c + 1) * (unsigned)(a.H / 2) / N);
    }
    __syncthreads();

    // weights prefetched one layer ahead: this wave's first router row or shared-expert unit, and
    // its first pass over the shared expert's down rows
    uint4 pr[RU];
    GuUnit pu;
    DnPass<ITERS> psd;

    for (int l = 0; l < L; ++l) {
        // Everything below is recomputed per layer from laundered thread and workgroup indices, so
        // the compiler does not hoist per-lane addresses out of the loop and keep them live.
        int tidv = threadIdx.x;
        asm volatile("" : "+v"(tidv));
        const int cs = blockIdx.x;
        const int tid = tidv, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6), ks = lane % KSUB;
        const int c = cs, N = gridDim.x;
        const int H = a.H, E = a.E, I = a.I, k = a.k, S = a.S;
        const int NB = H / kBlock, NI = I / kBlock, Hh = H / 2, Ih = I / 2;
        // LDS
        uint16_t* xr = (uint16_t*)smem;                       // [T][H] residual x_l
        uint16_t* xn = xr + T * H;                            // [T][H] MoE input (normalised) as bf16
        half2_t* xh = (half2_t*)(xn + T * H);                 // [T][H/2] its FP8 codes as f16
        float* lg = (float*)(xh + T * Hh);                    // [T][E] logits (rows of E rounded up to 4)
        half2_t* hqs = (half2_t*)(lg + T * ((E + 3) & ~3));   // [T][I/2] shared expert's FP8 h as f16
        half2_t* hqr = hqs + T * Ih;                          // [kMaxTokens][I/2] own routed expert's FP8 h
        float* dsh = (float*)(hqr + kMaxTokens * Ih);         // [T][rmax] shared down output, own rows
        float* dg = dsh + T * a.rmax;                         // [T][k][rmax] gathered routed down outputs
        float* cmax = dg + T * kMaxTopK * a.rmax;             // [kMaxTokens * I / 64] chunk maxima
        float* hsraw = cmax + kMaxTokens * I / 64;            // [T][I] shared expert's h (fp32)
        // per-workgroup ranges
        const int eA = __builtin_amdgcn_readfirstlane(s_rng[0]), eB = __builtin_amdgcn_readfirstlane(s_rng[1]);
        const int iA = __builtin_amdgcn_readfirstlane(s_rng[2]), iB = __builtin_amdgcn_readfirstlane(s_rng[3]);
        const int oA = __builtin_amdgcn_readfirstlane(s_rng[4]), oB = __builtin_amdgcn_readfirstlane(s_rng[5]);
        const int nro = oB - oA;
        const int nr = eB - eA, nu0 = nr + (iB - iA);
        const int sh_passes = S ? (nro + UPW - 1) / UPW : 0;

        const LayerPtrs Lw = a.layers[l];
        const uint16_t* router = (const uint16_t*)Lw.router;
        const uint4* w13 = (const uint4*)Lw.w13;
        const uint8_t* w13s = (const uint8_t*)Lw.w13s;
        const uint4* w2 = (const uint4*)Lw.w2;
        const uint8_t* w2s = (const uint8_t*)Lw.w2s;
        const uint32_t stamp = stamp_of(epoch, L, l);
        const int par = l & 1;
        w.layer = l;

        PK_MARK(0);
        const int u0 = wv;
        auto prefetch = [&](int lp) {
            const LayerPtrs P = a.layers[lp];
            if (u0 < nr) router_load((const uint16_t*)P.router, eA + u0, H, pr, lane);
            else if (u0 < nu0) gu_load((const uint4*)P.w13, (const uint8_t*)P.w13s, E, iA + u0 - nr, I, NB, pu, lane);
            if (wv < sh_passes)
                dn_load<KSUB, ITERS>((const uint4*)P.w2, (const uint8_t*)P.w2s, E,
                                     oA + min(wv * UPW + lane / KSUB, nro - 1), H, NI, psd, lane);
        };
        if (l == 0) prefetch(0);

        // ---- round X: the layer input
        if (l == 0) {
            for (int i = tid; i < T * H / 8; i += NTH) ((u32x4*)xr)[i] = gp((const u32x4*)a.x_in)[i];
        } else {
            const uint64_t* src = a.xw + (size_t)par * kMaxTokens * Hh;
            uint64_t v[Z::MX];
            w.code = 1;
            poll_issue<Z::MX>(src, tid, T * Hh, v);
            const bool ok = poll_wait<Z::MX>(src, tid, T * Hh, stamp, v, w);
#pragma unroll
            for (int m = 0; m < Z::MX; ++m) {
                const int i = tid + m * NTH;
                if (i < T * Hh) ((uint32_t*)xr)[i] = (uint32_t)v[m];
            }
            if (__syncthreads_or(!ok)) return;
        }
        __syncthreads();
        PK_MARK(1);
        if (a.trace) {
            GLOBAL uint16_t* tr = gp(a.trace) + (size_t)l * T * H;
            for (int i = tid; i < T * nro; i += NTH) {
                const int t = i / nro, r = oA + i - t * nro;
                tr[t * H + r] = xr[t * H + r];
            }
        }

        // ---- MoE input: optional RMSNorm (sum of squares in fp64), per-token FP8 quantisation.  Each
        // thread owns 4-element quads; one barrier joins the per-wave partial sums.  The maximum of
        // |bf16(x * r)| is bf16(max|x| * r) because rounding is monotonic.
        {
            const int NQ = H / 4;  // quads per token
            double ss[T];
            float mx[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                ss[t] = 0.0;
                mx[t] = 0.0f;
            }
            for (int i = tid; i < T * NQ; i += NTH) {
                int t = 0;
#pragma unroll
                for (int tt = 1; tt < T; ++tt) t += i >= tt * NQ ? 1 : 0;
                const uint2 v = ((const uint2*)xr)[i];
                double d = 0.0;
                float m = 0.0f;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint32_t w2 = q ? v.y : v.x;
                    const float x0 = bf16_to_f32(w2), x1 = bf16_to_f32(w2 >> 16);
                    m = fmaxf(m, fmaxf(fabsf(x0), fabsf(x1)));
                    d = fma((double)x0, (double)x0, d);
                    d = fma((double)x1, (double)x1, d);
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
                const double sv = a.normalize ? sum64(ss[t]) : 0.0;
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
                for (int q = 0; q < NWV; ++q) {
                    sv += redd[q * T + t];
                    mv = fmaxf(mv, redf[q * T + t]);
                }
                double r = 1.0;
                if (a.normalize) {
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
                sx[tid] = sv;
                if (a.x_scale && c == 0) gp(a.x_scale)[(size_t)l * T + tid] = sv;
            }
            for (int i = tid; i < T * NQ; i += NTH) {
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
                uint2 v = ((const uint2*)xr)[i];
                if (a.normalize) {
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
                uint32_t cd[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint32_t d = q ? v.y : v.x;
                    cd[q] = e4m3_pack2(bf16_to_f32(d) / sv, bf16_to_f32(d >> 16) / sv);
                    xh[i * 2 + q] = e4m3x2_to_f16x2(cd[q]);
                }
                if (a.x_codes && c == 0)
                    *(GLOBAL uint32_t*)(gp(a.x_codes) + (size_t)l * T * H + (size_t)i * 4) = cd[0] | (cd[1] << 16);
            }
            __syncthreads();
        }
        PK_MARK(2);
        // ---- router rows and shared-expert gate/up units, published (round R)
        for (int u = wv; u < nu0; u += NWV) {
            if (u < nr) {
                if (u != u0) router_load(router, eA + u, H, pr, lane);
                float acc[T];
                router_dot<T>(pr, H, xn, acc, lane);
                const int e = eA + u;
#pragma unroll
                for (int t = 0; t < T; ++t)
                    if (lane == t) astore64(a.lw + ((size_t)par * kMaxTokens + t) * E + e, word(acc[t], stamp));
            } else {
                const int i = iA + u - nr;
                if (u != u0) gu_load(w13, w13s, E, i, I, NB, pu, lane);
                int tok[T];
#pragma unroll
                for (int t = 0; t < T; ++t) tok[t] = t;
                float g[T], up[T];
                gu_dot<T>(pu, NB, xh, Hh, tok, T, g, up, lane);
#pragma unroll
                for (int t = 0; t < T; ++t)
                    if (lane == t)
                        astore64(a.shw + ((size_t)par * kMaxTokens + t) * I + i,
                                 word(swiglu(g[t] * sx[t], up[t] * sx[t]), stamp));
            }
        }

        PK_MARK(3);
        // ---- round R: logits and shared h; top-k; FP8 shared h
        {
            const uint64_t* lsrc = a.lw + (size_t)par * kMaxTokens * E;
            const uint64_t* ssrc = a.shw + (size_t)par * kMaxTokens * I;
            uint64_t vl[Z::ML], vs[Z::MS];
            poll_issue<Z::ML>(lsrc, tid, T * E, vl);
            if (S) poll_issue<Z::MS>(ssrc, tid, T * I, vs);
            w.code = 2;
            bool ok = poll_wait<Z::ML>(lsrc, tid, T * E, stamp, vl, w);
            if (ok && S) {
                w.code = 3;
                ok = poll_wait<Z::MS>(ssrc, tid, T * I, stamp, vs, w);
            }
            if (__syncthreads_or(!ok)) return;
            PK_MARK(4);
#pragma unroll
            for (int m = 0; m < Z::ML; ++m) {
                const int i = tid + m * NTH;
                if (i < T * E) lg[i] = payload(vl[m]);
            }
            if (S) {
#pragma unroll
                for (int m = 0; m < Z::MS; ++m) {
                    const int i = tid + m * NTH;
                    if (i < T * I) hsraw[i] = payload(vs[m]);
                }
            }
            __syncthreads();
            route_lds<T>(lg, E, k, &st, ids, wts, tid);
        }
        const int D = st.n;
        if (c == 0) {
            for (int i = tid; i < T * k; i += NTH) {
                if (a.ids_out) gp(a.ids_out)[(size_t)l * T * k + i] = ids[i];
                if (a.w_out) gp(a.w_out)[(size_t)l * T * k + i] = wts[i];
            }
        }
        if (tid < kMaxSlots) {  // own slot group: slot s owns workgroups [s*N/D, (s+1)*N/D)
            const int s = tid;
            const int gA = (int)((unsigned)(s * N) / (unsigned)D), gB = (int)((unsigned)((s + 1) * N) / (unsigned)D);
            if (s < D && c >= gA && c < gB) {
                s_grp[0] = s;
                s_grp[1] = gA;
            }
        }
        if (tid < kMaxSlots * kMaxTokens) {  // (token, rank) -> (slot, position)
            const int s = tid / kMaxTokens, j = tid % kMaxTokens;
            if (s < D && j < st.ntok[s]) {
                const int t = st.tok[s][j], r = st.rank[s][j];
                qs[t * k + r] = s;
                qj[t * k + r] = j;
            }
        }
        __syncthreads();
        const int ms = s_grp[0];
        const int ns = (int)((unsigned)((ms + 1) * N) / (unsigned)D) - s_grp[1], cc = c - s_grp[1];
        const int me = st.expert[ms], mnt = st.ntok[ms];
        int mtok[T];
#pragma unroll
        for (int q = 0; q < T; ++q) mtok[q] = q < mnt ? st.tok[ms][q] : 0;
        const int hA = (int)((unsigned)(cc * I) / (unsigned)ns), hB = (int)((unsigned)((cc + 1) * I) / (unsigned)ns);
        const int dA = (int)((unsigned)(cc * H) / (unsigned)ns), dB = (int)((unsigned)((cc + 1) * H) / (unsigned)ns);
        const int nd = dB - dA, rd_passes = (nd + UPW - 1) / UPW;

        PK_MARK(5);
        // ---- routed loads: gate/up units in two buffers, then the first down passes.  Every load
        // issued earlier (the prefetch) has long completed; waiting for them here keeps the shared
        // expert's work below from waiting for the routed loads.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        const int nu = hB - hA > wv ? (hB - hA - wv + NWV - 1) / NWV : 0;  // units of this wave
        const int ulast = nu > 0 ? hA + wv + (nu - 1) * NWV : hA;
        auto unit_i = [&](int m) { return min(hA + wv + m * NWV, ulast); };
        GuUnit ga[DG], gb[DG];
#pragma unroll
        for (int q = 0; q < DG; ++q) gu_load(w13, w13s, me, unit_i(q), I, NB, ga[q], lane);
#pragma unroll
        for (int q = 0; q < DG; ++q) gu_load(w13, w13s, me, unit_i(DG + q), I, NB, gb[q], lane);
        const int ndp = rd_passes > wv ? (rd_passes - wv + NWV - 1) / NWV : 0;  // routed down passes of this wave
        DnPass<ITERS> dp[Z::DPM];
#pragma unroll
        for (int m = 0; m < Z::DPM; ++m) {
            const int g = wv + min(m, max(ndp - 1, 0)) * NWV;
            dn_load<KSUB, ITERS>(w2, w2s, me, dA + min(g * UPW + lane / KSUB, max(nd - 1, 0)), H, NI, dp[m], lane);
        }

        // ---- shared expert: FP8 requantisation of its h, its down rows (own rows, every token) into
        // LDS, while the routed weights are in flight
        if (S) {
            float hv[Z::MS];
#pragma unroll
            for (int m = 0; m < Z::MS; ++m) hv[m] = hsraw[min(tid + m * NTH, T * I - 1)];
            requant<Z::MS>(hv, tid, T, I, shs, (_Float16*)hqs, cmax);
            __syncthreads();
        }
        for (int g = wv; g < sh_passes; g += NWV) {
            if (g != wv) dn_load<KSUB, ITERS>(w2, w2s, E, oA + min(g * UPW + lane / KSUB, nro - 1), H, NI, psd, lane);
            float o[T];
            dn_dot<KSUB, ITERS, T>(psd, hqs, Ih, T, o, lane);
            const int v = g * UPW + lane / KSUB;
            if (ks == 0 && v < nro) {
#pragma unroll
                for (int t = 0; t < T; ++t) dsh[t * a.rmax + v] = o[t] * shs[t];
            }
        }

        // ---- routed gate/up: compute from one buffer while the other is in flight
        auto gu_unit = [&](const GuUnit& u, int m) {
            float g[T], up[T];
            gu_dot<T>(u, NB, xh, Hh, mtok, mnt, g, up, lane);
            const int i = hA + wv + m * NWV;
#pragma unroll
            for (int q = 0; q < T; ++q)
                if (q < mnt && lane == q)
                    astore64(a.hw + (((size_t)par * kMaxSlots + ms) * kMaxTokens + q) * I + i,
                             word(swiglu(g[q] * sx[mtok[q]], up[q] * sx[mtok[q]]), stamp));
        };
        for (int m0 = 0; m0 < nu; m0 += 2 * DG) {
#pragma unroll
            for (int q = 0; q < DG; ++q)
                if (m0 + q < nu) gu_unit(ga[q], m0 + q);
            if (m0 + 2 * DG < nu) {
#pragma unroll
                for (int q = 0; q < DG; ++q) gu_load(w13, w13s, me, unit_i(m0 + 2 * DG + q), I, NB, ga[q], lane);
            }
#pragma unroll
            for (int q = 0; q < DG; ++q)
                if (m0 + DG + q < nu) gu_unit(gb[q], m0 + DG + q);
            if (m0 + 3 * DG < nu) {
#pragma unroll
                for (int q = 0; q < DG; ++q) gu_load(w13, w13s, me, unit_i(m0 + 3 * DG + q), I, NB, gb[q], lane);
            }
        }

        PK_MARK(6);
        PK_MARK(7);
        // ---- round H: own expert's h, FP8 requantisation
        {
            const uint64_t* src = a.hw + ((size_t)par * kMaxSlots + ms) * kMaxTokens * I;
            uint64_t v[Z::MH];
            poll_issue<Z::MH>(src, tid, mnt * I, v);
            w.code = 4;
            const bool ok = poll_wait<Z::MH>(src, tid, mnt * I, stamp, v, w);
            if (__syncthreads_or(!ok)) return;
            PK_MARK(8);
            float hv[Z::MH];
#pragma unroll
            for (int m = 0; m < Z::MH; ++m) hv[m] = payload(v[m]);
            requant<Z::MH>(hv, tid, mnt, I, rhs, (_Float16*)hqr, cmax);
            __syncthreads();
        }

        // ---- routed down rows of the own expert, published unweighted (round D)
        auto dn_pass = [&](const DnPass<ITERS>& d, int g) {
            float o[T];
            dn_dot<KSUB, ITERS, T>(d, hqr, Ih, mnt, o, lane);
            const int v = g * UPW + lane / KSUB;
            if (ks == 0 && v < nd) {
#pragma unroll
                for (int q = 0; q < T; ++q)
                    if (q < mnt)
                        astore64(a.dw + (((size_t)par * kMaxSlots + ms) * kMaxTokens + q) * H + dA + v,
                                 word(o[q] * rhs[q], stamp));
            }
        };
#pragma unroll
        for (int m = 0; m < Z::DPM; ++m)
            if (m < ndp) dn_pass(dp[m], wv + m * NWV);
        for (int m = Z::DPM; m < ndp; ++m) {
            const int g = wv + m * NWV;
            dn_load<KSUB, ITERS>(w2, w2s, me, dA + min(g * UPW + lane / KSUB, nd - 1), H, NI, dp[0], lane);
            dn_pass(dp[0], g);
        }

        PK_MARK(9);
        // ---- round D: the k routed terms of every token for the own rows; combine; next input
        {
            const int n = T * k * nro;  // word (t, r, v)
            for (int b = 0; b < n; b += Z::MG * NTH) {
                uint64_t v[Z::MG];
                const uint64_t* src[Z::MG];
#pragma unroll
                for (int m = 0; m < Z::MG; ++m) {
                    const int i = min(b + tid + m * NTH, n - 1);
                    const int tr = i / nro, r = i - tr * nro;  // tr = t * k + rank
                    const int s = qs[tr], j = qj[tr];
                    src[m] = a.dw + (((size_t)par * kMaxSlots + s) * kMaxTokens + j) * H + oA + r;
                    v[m] = aload64(src[m]);
                }
                w.code = 5;
                const long long t0 = wall_clock64();
                bool ok = true;
                for (int it = 0;; ++it) {
                    bool done = true;
#pragma unroll
                    for (int m = 0; m < Z::MG; ++m)
                        done &= (b + tid + m * NTH >= n) || (uint32_t)(v[m] >> 32) == stamp;
                    if (done) break;
                    if ((it & 7) == 7) {
                        if (aload32(a.ctl + C_ABORT) != 0u) {
                            ok = false;
                            break;
                        }
                        if (wall_clock64() - t0 > a.timeout) {
                            raise_abort(w);
                            ok = false;
                            break;
                        }
                    }
                    __builtin_amdgcn_s_sleep(1);
#pragma unroll
                    for (int m = 0; m < Z::MG; ++m)
                        if (b + tid + m * NTH < n && (uint32_t)(v[m] >> 32) != stamp) v[m] = aload64(src[m]);
                }
                if (__syncthreads_or(!ok)) return;
#pragma unroll
                for (int m = 0; m < Z::MG; ++m) {
                    const int i = b + tid + m * NTH;
                    if (i < n) {
                        const int tr = i / nro, r = i - tr * nro;
                        dg[tr * a.rmax + r] = payload(v[m]);
                    }
                }
            }
            __syncthreads();
            PK_MARK(10);
            if (l + 1 < L) prefetch(l + 1);
            const bool last = l == L - 1;
            const uint32_t nstamp = stamp_of(epoch, L, l + 1);
            uint64_t* xdst = a.xw + (size_t)(par ^ 1) * kMaxTokens * Hh;
            for (int i0 = 0; i0 < T * nro; i0 += NTH) {  // uniform loop: thread (token, row), rows in pairs
                const int i = i0 + tid;
                const bool act = i < T * nro;
                const int t = act ? (int)((unsigned)i / (unsigned)nro) : 0, v = act ? i - t * nro : 0;
                float dv[kMaxTopK];
#pragma unroll
                for (int r = 0; r < kMaxTopK; ++r) dv[r] = r < k ? dg[(t * k + r) * a.rmax + v] : 0.0f;
                float y = 0.0f;
#pragma unroll
                for (int r = 0; r < kMaxTopK; ++r)
                    if (r < k) y = fmaf(wts[t * k + r], dv[r], y);
                if (S) y += dsh[t * a.rmax + v];
                const int row = oA + v;
                const uint32_t xb = f32_to_bf16(bf16_to_f32(xr[t * H + row]) + y);
                const uint32_t other = xchg<0>(xb);  // the neighbouring row (nro is even: pairs stay in a lane pair)
                if (act) {
                    if (last && a.y) gp(a.y)[(size_t)t * H + row] = y;
                    if ((v & 1) == 0) {
                        const uint32_t pairv = xb | (other << 16);
                        if (!last) astore64(xdst + (size_t)t * Hh + row / 2, ((uint64_t)nstamp << 32) | pairv);
                        else if (a.x_out) *(GLOBAL uint32_t*)(gp(a.x_out) + (size_t)t * H + row) = pairv;
                    }
                }
            }
        }
        PK_MARK(11);
    }

    // end of pass: once every workgroup has arrived (each read the epoch first), advance it
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const long long t0 = wall_clock64();
        bool ok = true;
        while (aload32(a.ctl + C_ARRIVE) < gridDim.x) {
            if (aload32(a.ctl + C_ABORT) != 0u || wall_clock64() - t0 > a.timeout) {
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (ok) {
            astore32(a.ctl + C_ARRIVE, 0u);
            astore32(a.ctl + C_EPOCH, epoch + 1u);
        } else {
            w.code = 6;
            raise_abort(w);
        }
    }
}

// ------------------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------------------

size_t lds_bytes(const Shape& sh, int T, int rmax) {
    const size_t H = sh.H, E = sh.E, I = sh.I;
    return (size_t)T * H * 2 * 2 + (size_t)T * H * 2 + (size_t)T * ((E + 3) & ~3) * 4 + (size_t)T * I * 2 +
           (size_t)kMaxTokens * I * 2 + (size_t)T * rmax * 4 + (size_t)T * kMaxTopK * rmax * 4 +
           (size_t)kMaxTokens * I / 64 * 4 + (size_t)T * I * 4;
}

int grid_size(const Shape& sh, int cus) {
    int n = cus;
    n = n < sh.E ? n : sh.E;
    n = n < sh.H / 2 ? n : sh.H / 2;
    n = n < sh.I * sh.k ? n : sh.I * sh.k;
    return n;
}

int rows_max(const Shape& sh, int n) { return 2 * ((sh.H / 2 + n - 1) / n); }

template <int T, int KSUB, int ITERS>
static const void* kernel_ptr() {
    return (const void*)stack_kernel<T, KSUB, ITERS>;
}

static const void* pick_kernel(const Shape& sh, int T) {
    const int ks = sh.ksub(), it = sh.iters();
#define PK_CASE(TT)                                                              \
    if (T == TT) {                                                               \
        if (ks == 8 && it == 3) return kernel_ptr<TT, 8, 3>();                   \
        if (ks == 8 && it == 1) return kernel_ptr<TT, 8, 1>();                   \
        if (ks == 4 && it == 1) return kernel_ptr<TT, 4, 1>();                   \
        if (ks == 2 && it == 1) return kernel_ptr<TT, 2, 1>();                   \
    }
    PK_CASE(1)
    PK_CASE(2)
    PK_CASE(3)
    PK_CASE(4)
#undef PK_CASE
    return nullptr;
}

hipError_t check_resident(const Shape& sh, int T, int n, int* max_per_cu) {
    const void* f = pick_kernel(sh, T);
    if (!f) return hipErrorInvalidValue;
    const size_t lds = lds_bytes(sh, T, rows_max(sh, n));
    hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, NTH, lds);
    if (max_per_cu) *max_per_cu = nb;
    return e;
}

hipError_t launch_stack(const Shape& sh, int T, int n, const StackArgs& args, hipStream_t stream) {
    const void* f = pick_kernel(sh, T);
    if (!f) return hipErrorInvalidValue;
    StackArgs a = args;
    void* params[] = {&a};
    return hipLaunchCooperativeKernel(f, dim3(n), dim3(NTH), params, lds_bytes(sh, T, a.rmax), stream);
}

}  // namespace pk
}  // namespace moe
