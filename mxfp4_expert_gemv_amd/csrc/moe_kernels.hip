// moe_kernels.hip -- gfx950 kernels of the W4A8 sparse-MoE decode step.
//
// One layer is three launches (replayed from a HIP graph by the library), plus two small ones at
// 3-4 tokens:
//   k0_input          (3-4 tokens) one workgroup per token: RMSNorm of the residual and the FP8
//                     quantisation of the MoE input, once per layer.
//   k1_router         router GEMV, one wave per expert row (bf16 x bf16 products, fp32 FMA).  At
//                     1-2 tokens every workgroup also normalises the input itself and stores the
//                     FP8 codes of its share of it; at 3-4 tokens extra workgroups compute the
//                     shared expert's gate/up tiles (VALU form: one workgroup per tile and token),
//                     and above 3 tokens (2 in the matrix-core form) the last router workgroup
//                     to finish takes the top-k once (arrival ticket).
//   k2_gateup         the routed gate/up tiles (and at 1-2 tokens the shared expert's): at 1-3
//                     tokens (1-2 in the matrix-core form) every routed workgroup redoes the top-k from the logits (1-4 waves per
//                     token, lower index first on ties) and builds the list of distinct routed
//                     experts; each workgroup streams its 32-row MXFP4 gate/up tile: E2M1 pairs are
//                     converted to f16 in VGPRs and dot2-multiplied with the FP8 activation codes
//                     (as f16) held in LDS; writes h = SiLU(gate) * up and the tile's max |h|.
//   kq_requant        (3-4 tokens) the FP8 requantisation of every h vector, once per layer.
//   k3_down           one workgroup per 8-row output tile, over every routed expert and the shared
//                     one: requantises each (token, expert) h vector to FP8 in LDS (or decodes its
//                     codes), streams the MXFP4 down rows and sums the routing-weighted results in
//                     a fixed order (no float atomics); writes y and the bf16 residual.
//
// What is computed follows the MoE decode step described on the pages (tanhow.com, "NVIDIA 在单台
// DGX Spark 上叠加三项优化..." sections "Ling 3.0 是什么" (8 of 512 routed experts + 1 shared) and
// "三项优化是什么" items 1 and 3 (width-768 MXFP4 experts; a 4-position verify touching up to 32
// experts); devotd.net "dgx-spark-moe-inference-optimizations" section 2 (MXFP4 = blocked 4-bit
// float, 4-bit weights with 8-bit activations)).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <string>

#include "moe_kernels.h"
#include "moe_launch.h"

MOE_KERNELS_NS_BEGIN

// The repack kernels, the grid sizes of the timing record and the run-time compiled kernel names
// belong to the shape-generic build only; a build with the shape folded in (MOE_SHAPE_H defined)
// contributes its layer launcher.
#ifndef MOE_SHAPE_H

// ------------------------------------------------------------------------------------------------
// repack kernels (canonical row-major -> lane tiles; pure permutations of 16-byte units / bytes)
// ------------------------------------------------------------------------------------------------

__device__ __forceinline__ int gu_row(int lane, int tile, int I) {
    const int r = lane >> 1;
    return r < kGuOut ? tile * kGuOut + r : I + tile * kGuOut + r - kGuOut;
}

__global__ void repack_w13(const uint4* __restrict__ src, uint4* __restrict__ dst, int nexp, int I, int H, int bpl) {
    const int NB = H / kBlock, GW = NB / (2 * bpl), tiles = I / kGuOut;
    const uint64_t total = (uint64_t)nexp * tiles * GW * bpl * kWave;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        uint64_t r = u / kWave;
        const int step = (int)(r % bpl);
        r /= bpl;
        const int w = (int)(r % GW);
        r /= GW;
        const int tile = (int)(r % tiles);
        const uint64_t e = r / tiles;
        const int c = (w * bpl + step) * 2 + (lane & 1);
        dst[u] = src[(e * 2 * I + gu_row(lane, tile, I)) * NB + c];
    }
}

__global__ void repack_w13s(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int nexp, int I, int H,
                            int bpl) {
    const int NB = H / kBlock, GW = NB / (2 * bpl), tiles = I / kGuOut;
    const uint64_t total = (uint64_t)nexp * tiles * GW * kWave * bpl;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int step = (int)(u % bpl);
        uint64_t r = u / bpl;
        const int lane = (int)(r % kWave);
        r /= kWave;
        const int w = (int)(r % GW);
        r /= GW;
        const int tile = (int)(r % tiles);
        const uint64_t e = r / tiles;
        const int c = (w * bpl + step) * 2 + (lane & 1);
        dst[u] = src[(e * 2 * I + gu_row(lane, tile, I)) * NB + c];
    }
}

// Matrix-core layout (MOE_F_MFMA).  w13: the same [E+S][I/16][GW][BPL][64 lanes][16 B] units, but
// unit `step` of lane l holds, in dword q, the 8 codes of row (step < BPL/2 ? gate : up) row
// 16 tile + l % 16, block w 2 BPL + 4 (step % (BPL/2)) + q, K 8 (l / 16) .. +8 (bytes 4 (l / 16)
// .. +4 of that block): a permutation of dwords.  w13_s: [E+S][I/16][GW][16 rows][4 BPL] bytes,
// row r's gate scales of the wave's 2 BPL blocks, then its up scales (the four lanes of a row
// read the same 4 BPL bytes).
__global__ void repack_w13_mf(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, int nexp, int I, int H,
                              int bpl) {
    const int NB = H / kBlock, GW = NB / (2 * bpl), tiles = I / kGuOut, RD = H / 8;  // dwords per row
    const uint64_t total = (uint64_t)nexp * tiles * GW * bpl * kWave * 4;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int q = (int)(u % 4);
        uint64_t r = u / 4;
        const int lane = (int)(r % kWave);
        r /= kWave;
        const int step = (int)(r % bpl);
        r /= bpl;
        const int w = (int)(r % GW);
        r /= GW;
        const int tile = (int)(r % tiles);
        const uint64_t e = r / tiles;
        const int half = bpl / 2, gu = step / half;
        const int row = gu * I + tile * kGuOut + (lane & 15);
        const int blk = w * 2 * bpl + 4 * (step - gu * half) + q;
        dst[u] = src[(e * 2 * I + row) * RD + blk * 4 + (lane >> 4)];
    }
}

__global__ void repack_w13s_mf(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int nexp, int I, int H,
                               int bpl) {
    const int NB = H / kBlock, BW = 2 * bpl, GW = NB / BW, tiles = I / kGuOut;
    const uint64_t total = (uint64_t)nexp * tiles * GW * 16 * 2 * BW;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int k = (int)(u % (2 * BW));
        uint64_t r = u / (2 * BW);
        const int rr = (int)(r % 16);
        r /= 16;
        const int w = (int)(r % GW);
        r /= GW;
        const int tile = (int)(r % tiles);
        const uint64_t e = r / tiles;
        const int gu = k / BW, j = k - gu * BW;
        dst[u] = src[(e * 2 * I + gu * I + tile * kGuOut + rr) * NB + w * BW + j];
    }
}

__global__ void repack_w2(const uint4* __restrict__ src, uint4* __restrict__ dst, int nexp, int H, int I, int ksub) {
    const int NI = I / kBlock, R = kWave / ksub, iters = NI / ksub, tiles = H / R;
    const uint64_t total = (uint64_t)nexp * tiles * iters * kWave;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        uint64_t r = u / kWave;
        const int it = (int)(r % iters);
        r /= iters;
        const int tile = (int)(r % tiles);
        const uint64_t e = r / tiles;
        dst[u] = src[(e * H + tile * R + lane / ksub) * NI + it * ksub + lane % ksub];
    }
}

__global__ void repack_w2s(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int nexp, int H, int I,
                           int ksub) {
    const int NI = I / kBlock, R = kWave / ksub, iters = NI / ksub, tiles = H / R;
    const uint64_t total = (uint64_t)nexp * tiles * iters * kWave;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
         u += (uint64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(u % kWave);
        uint64_t r = u / kWave;
        const int it = (int)(r % iters);
        r /= iters;
        const int tile = (int)(r % tiles);
        const uint64_t e = r / tiles;
        dst[u] = src[(e * H + tile * R + lane / ksub) * NI + it * ksub + lane % ksub];
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
                         bool mfma, hipStream_t stream) {
    const int nexp = sh.E + sh.S;
    const unsigned B = 256;
    hipError_t e = hipMemcpyAsync(d_router, router, sh.router_bytes(), hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return e;
    if (mfma) {
        repack_w13_mf<<<grid_for((uint64_t)nexp * sh.I * sh.H / 4, B), B, 0, stream>>>(
            (const uint32_t*)w13, (uint32_t*)d_w13, nexp, sh.I, sh.H, sh.bpl());
        repack_w13s_mf<<<grid_for((uint64_t)nexp * 2 * sh.I * sh.H / 32, B), B, 0, stream>>>(
            (const uint8_t*)w13s, (uint8_t*)d_w13s, nexp, sh.I, sh.H, sh.bpl());
    } else {
        repack_w13<<<grid_for((uint64_t)nexp * sh.I * sh.H / 16, B), B, 0, stream>>>(
            (const uint4*)w13, (uint4*)d_w13, nexp, sh.I, sh.H, sh.bpl());
        repack_w13s<<<grid_for((uint64_t)nexp * 2 * sh.I * sh.H / 32, B), B, 0, stream>>>(
            (const uint8_t*)w13s, (uint8_t*)d_w13s, nexp, sh.I, sh.H, sh.bpl());
    }
    repack_w2<<<grid_for((uint64_t)nexp * sh.H * sh.I / 32, B), B, 0, stream>>>(
        (const uint4*)w2, (uint4*)d_w2, nexp, sh.H, sh.I, sh.ksub());
    repack_w2s<<<grid_for((uint64_t)nexp * sh.H * sh.I / 32, B), B, 0, stream>>>(
        (const uint8_t*)w2s, (uint8_t*)d_w2s, nexp, sh.H, sh.I, sh.ksub());
    return hipGetLastError();
}

#endif  // MOE_SHAPE_H

static int routed_slots_max(const Shape& sh, int T) { return T * sh.k < sh.E ? T * sh.k : sh.E; }

#ifndef MOE_SHAPE_H
__global__ void clear_u64(unsigned long long* p, uint64_t n) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = 0ull;
}

hipError_t launch_clear_u64(unsigned long long* p, uint64_t n, hipStream_t stream) {
    clear_u64<<<grid_for(n, 256), 256, 0, stream>>>(p, n);
    return hipGetLastError();
}
#endif  // MOE_SHAPE_H

// Launch decisions shared by the ahead-of-time launcher and the list of kernels compiled at run time.
// Top-k waves per token in the 1-2 token gate/up workgroups (workgroups of at least T W waves).
static int gateup_wt(const Shape& sh, int T) {
    const int wt = T == 1 ? 4 : T == 2 ? 2 : 1;
    return sh.gw() >= T * wt ? wt : 1;
}
// 3-4 tokens: the down kernel runs two workgroups per CU (each SIMD then holds twice the waves that
// hide the LDS latency of its dot phase), with two unit groups per wave.
static bool down_two_per_cu(const Shape& sh, int T) { return T >= 3 && sh.H % (2 * kDownGrid) == 0; }

#ifndef MOE_SHAPE_H
int layer_grid(const Shape& sh, int T, int kind) {
    const bool central = T >= 3;
    const int tiles = sh.gu_tiles(), n_router_wg = (sh.E + sh.gw() - 1) / sh.gw();
    switch (kind) {
        case kKernInput: return central ? T : 0;
        case kKernRouter: return n_router_wg + (central ? sh.S * tiles * T : 0);  // at most (MFMA form: S tiles)
        case kKernGateup: return (central ? 0 : sh.S * tiles) + routed_slots_max(sh, T) * tiles;
        case kKernRequant: return T >= kKqMinT ? sh.pairs(T) : 0;
        case kKernDown: return down_two_per_cu(sh, T) ? 2 * kDownGrid : kDownGrid;
        default: return 0;
    }
}

bool jit_kernel_names(const Shape& sh, int T, bool mfma, std::string (&names)[kLayerKernels]) {
    if (T < 1 || T > kMaxTokens || !shape_supported(sh)) return false;
    const std::string t = std::to_string(T), bpl = std::to_string(sh.bpl()), mf = mfma ? "true" : "false";
    names[kKernInput] = T >= 3 ? "moe::k0_input<false>" : "";
    names[kKernRouter] = "moe::k1_router<" + t + ", " + bpl + ", " + mf + ">";
    names[kKernGateup] =
        "moe::k2_gateup<" + t + ", " + bpl + ", " + std::to_string(gateup_wt(sh, T)) + ", " + mf + ">";
    names[kKernRequant] = T >= kKqMinT ? "moe::kq_requant<false>" : "";
    names[kKernDown] = "moe::k3_down<" + std::to_string(sh.ksub()) + ", " + std::to_string(sh.iters()) + ", " + t +
                       ", " + std::to_string(down_two_per_cu(sh, T) ? 2 : T) + ">";
    return true;
}
#endif  // MOE_SHAPE_H

// One kernel launch: the ahead-of-time instance kern, or the run-time compiled function jf when there
// is one; in timing mode (ev) a launch whose start/stop events carry the kernel's own begin and end.
template <typename Kern, typename Args>
static hipError_t launch(Kern kern, hipFunction_t jf, unsigned grid, unsigned block, size_t lds, hipStream_t stream,
                         hipEvent_t* ev, const Args& a) {
    if (jf) {
        void* params[] = {(void*)&a};
        if (ev)
            return hipExtModuleLaunchKernel(jf, grid * block, 1, 1, block, 1, 1, lds, stream, params, nullptr, ev[0],
                                            ev[1], 0);
        return hipModuleLaunchKernel(jf, grid, 1, 1, block, 1, 1, (unsigned)lds, stream, params, nullptr);
    }
    if (ev)
        hipExtLaunchKernelGGL(kern, dim3(grid), dim3(block), (uint32_t)lds, stream, ev[0], ev[1], 0u, a);
    else
        kern<<<grid, block, lds, stream>>>(a);
    return hipGetLastError();
}

#define MOE_TRY(x)                          \
    do {                                    \
        const hipError_t e_ = (x);          \
        if (e_ != hipSuccess) return e_;    \
    } while (0)

template <int T, int BPL, int KSUB, int ITERS, bool STAMP>
static hipError_t launch_layer_t(const Shape& sh, const LayerPtrs& L, const RunPtrs& P, bool normalize,
                                 hipStream_t stream, hipEvent_t* ev, const JitKernels* jit) {
    const int GW = sh.gw(), tiles = sh.gu_tiles(), R = sh.down_rows();
    constexpr bool CENTRAL = T >= 3;  // input and h requantisation once per layer (k0, kq)
    auto jf = [&](int kind) -> hipFunction_t { return jit ? jit->fn[T - 1][kind] : nullptr; };
    auto evk = [&](int kind) -> hipEvent_t* { return ev ? ev + 2 * kind : nullptr; };
    if (CENTRAL) {
        K0Args a0{P.x, P.xn, P.xq, P.xs, P.trace, P.x_scale, P.x_codes, sh.H, normalize ? 1 : 0};
        a0.stamp = P.stamp[kKernInput];
        MOE_TRY(launch(k0_input<STAMP>, jf(kKernInput), T, 1024, (size_t)sh.H * 2, stream, evk(kKernInput), a0));
    }
    const int n_router_wg = (sh.E + GW - 1) / GW;
    // shared gate/up items in the router kernel: per tile, or per tile and token
    const int n_sh1 = CENTRAL ? sh.S * tiles * (L.w13_mfma ? 1 : T) : 0;
    const bool ticket = T > gu_route_max_t(L.w13_mfma);  // the router kernel takes the top-k
    K1Args a1{(const uint16_t*)L.router, P.x, P.xn, P.xq, P.xs, CENTRAL ? nullptr : P.trace,
              CENTRAL ? nullptr : P.x_scale, CENTRAL ? nullptr : P.x_codes, P.logits, P.ticket, P.slots,
              ticket ? P.ids : nullptr, ticket ? P.w : nullptr, (const uint4*)L.w13, (const uint8_t*)L.w13s, P.h,
              P.hamax, sh.H, sh.E, sh.k, sh.S, sh.I, normalize ? 1 : 0, n_router_wg, T};
    a1.stamp = P.stamp[kKernRouter];
    const size_t lds1 = (size_t)T * sh.H * 2;
    if (L.w13_mfma)
        MOE_TRY(launch(k1_router<T, BPL, true, STAMP>, jf(kKernRouter), n_router_wg + n_sh1, 64 * GW, lds1, stream,
                       evk(kKernRouter), a1));
    else
        MOE_TRY(launch(k1_router<T, BPL, false, STAMP>, jf(kKernRouter), n_router_wg + n_sh1, 64 * GW, lds1, stream,
                       evk(kKernRouter), a1));

    const int n_sh_wg = CENTRAL ? 0 : sh.S * tiles;  // 1-2 tokens: shared gate/up tiles here
    const int n_gu_wg = routed_slots_max(sh, T) * tiles;
    K2Args a2{P.logits, P.xq, P.xs, (const uint4*)L.w13, (const uint8_t*)L.w13s, P.h, P.hamax, P.slots,
              ticket ? nullptr : P.ids, ticket ? nullptr : P.w, sh.H, sh.E, sh.k, sh.S, sh.I, n_sh_wg, T};
    a2.stamp = P.stamp[kKernGateup];
    const size_t lds2 = (size_t)T * sh.H * 2;
    constexpr int WT = T == 1 ? 4 : T == 2 ? 2 : 1;
    const int n2 = n_sh_wg + n_gu_wg;
    const bool wt = gateup_wt(sh, T) == WT;
    if (L.w13_mfma && wt)
        MOE_TRY(launch(k2_gateup<T, BPL, WT, true, STAMP>, jf(kKernGateup), n2, 64 * GW, lds2, stream,
                       evk(kKernGateup), a2));
    else if (L.w13_mfma)
        MOE_TRY(launch(k2_gateup<T, BPL, 1, true, STAMP>, jf(kKernGateup), n2, 64 * GW, lds2, stream,
                       evk(kKernGateup), a2));
    else if (wt)
        MOE_TRY(launch(k2_gateup<T, BPL, WT, false, STAMP>, jf(kKernGateup), n2, 64 * GW, lds2, stream,
                       evk(kKernGateup), a2));
    else
        MOE_TRY(launch(k2_gateup<T, BPL, 1, false, STAMP>, jf(kKernGateup), n2, 64 * GW, lds2, stream,
                       evk(kKernGateup), a2));

    if (T >= kKqMinT) {
        KQArgs aq{P.h, P.hamax, P.hq, P.hs, sh.I};
        aq.stamp = P.stamp[kKernRequant];
        MOE_TRY(launch(kq_requant<STAMP>, jf(kKernRequant), sh.pairs(T), 256, 0, stream, evk(kKernRequant), aq));
    }
    // down: one workgroup per CU-sized share of the rows (or two per CU, above); (slot, row) units
    // spread over up to 12 waves, UPW groups of 64 / KSUB units per wave
    const bool two_per_cu = down_two_per_cu(sh, T);
    const int dgrid = two_per_cu ? 2 * kDownGrid : kDownGrid, upw = two_per_cu ? 2 : T;
    const int rows = sh.H / dgrid;
    const int units_max = (routed_slots_max(sh, T) + sh.S * T) * rows, groups = (units_max + R - 1) / R;
    const int nw = std::max(std::min(groups, 12), 2);  // >= 2: slot list copy
    if (nw * upw < groups) return hipErrorInvalidValue;
    K3Args a3{P.slots, (const uint4*)L.w2, (const uint8_t*)L.w2s, P.h, P.hamax, P.hq, P.hs, P.xnext ? P.x : nullptr,
              P.xnext, P.y, sh.H, sh.E, sh.k, sh.S, sh.I, rows, units_max};
    a3.stamp = P.stamp[kKernDown];
    const size_t lds3 = (size_t)sh.pairs(T) * sh.I * 2 + (size_t)units_max * T * 4;
    if (two_per_cu)
        MOE_TRY(launch(k3_down<KSUB, ITERS, T, 2, STAMP>, jf(kKernDown), dgrid, 64 * nw, lds3, stream, evk(kKernDown),
                       a3));
    else
        MOE_TRY(launch(k3_down<KSUB, ITERS, T, T, STAMP>, jf(kKernDown), dgrid, 64 * nw, lds3, stream, evk(kKernDown),
                       a3));
    return hipSuccess;
}

template <int T, int BPL, bool STAMP>
static hipError_t launch_layer_s(const Shape& sh, const LayerPtrs& L, const RunPtrs& P, bool normalize,
                                 hipStream_t stream, hipEvent_t* ev, const JitKernels* jit) {
    const int ks = sh.ksub(), it = sh.iters();
#ifdef MOE_FIXED_KSUB  // a build for one shape: only its down-kernel geometry
    if (ks == MOE_FIXED_KSUB && it == MOE_FIXED_ITERS)
        return launch_layer_t<T, BPL, MOE_FIXED_KSUB, MOE_FIXED_ITERS, STAMP>(sh, L, P, normalize, stream, ev, jit);
#else
    if (ks == 8 && it == 3) return launch_layer_t<T, BPL, 8, 3, STAMP>(sh, L, P, normalize, stream, ev, jit);
    if (ks == 8 && it == 1) return launch_layer_t<T, BPL, 8, 1, STAMP>(sh, L, P, normalize, stream, ev, jit);
    if (ks == 4 && it == 1) return launch_layer_t<T, BPL, 4, 1, STAMP>(sh, L, P, normalize, stream, ev, jit);
    if (ks == 2 && it == 1) return launch_layer_t<T, BPL, 2, 1, STAMP>(sh, L, P, normalize, stream, ev, jit);
#endif
    return hipErrorInvalidValue;
}

// The stamped instances (timing record, mode 1) are the ahead-of-time ones: the run-time compiled
// module holds only the instances of normal runs.
template <int T, int BPL>
static hipError_t launch_layer_b(const Shape& sh, const LayerPtrs& L, const RunPtrs& P, bool normalize,
                                 hipStream_t stream, hipEvent_t* ev, const JitKernels* jit) {
    if (P.stamp[kKernRouter]) return launch_layer_s<T, BPL, true>(sh, L, P, normalize, stream, ev, nullptr);
    return launch_layer_s<T, BPL, false>(sh, L, P, normalize, stream, ev, jit);
}

template <int T>
static hipError_t launch_layer_tt(const Shape& sh, const LayerPtrs& L, const RunPtrs& P, bool normalize,
                                  hipStream_t stream, hipEvent_t* ev, const JitKernels* jit) {
#ifdef MOE_FIXED_BPL  // a build for one shape: only its gate/up geometry
    return sh.bpl() == MOE_FIXED_BPL ? launch_layer_b<T, MOE_FIXED_BPL>(sh, L, P, normalize, stream, ev, jit)
                                     : hipErrorInvalidValue;
#else
    return sh.bpl() == 8 ? launch_layer_b<T, 8>(sh, L, P, normalize, stream, ev, jit)
                         : launch_layer_b<T, 4>(sh, L, P, normalize, stream, ev, jit);
#endif
}

hipError_t launch_layer(const Shape& sh, int T, const LayerPtrs& L, const RunPtrs& P, bool normalize,
                        hipStream_t stream, hipEvent_t* ev, const JitKernels* jit) {
    switch (T) {
        case 1: return launch_layer_tt<1>(sh, L, P, normalize, stream, ev, jit);
        case 2: return launch_layer_tt<2>(sh, L, P, normalize, stream, ev, jit);
        case 3: return launch_layer_tt<3>(sh, L, P, normalize, stream, ev, jit);
        case 4: return launch_layer_tt<4>(sh, L, P, normalize, stream, ev, jit);
        default: return hipErrorInvalidValue;
    }
}

#ifndef MOE_SHAPE_H
bool shape_supported(const Shape& sh) {
    if (sh.H % 256 || sh.H > 2560 || sh.I % kBlock) return false;
    if (sh.gw() < 1 || sh.gw() > kMaxWaves) return false;
    const int ks = sh.ksub(), it = sh.iters();
    if (ks * it != sh.NI() || sh.NB() != sh.gw() * sh.bpl() * 2) return false;
    return (ks == 8 && (it == 1 || it == 3)) || (ks == 4 && it == 1) || (ks == 2 && it == 1);
}

#endif  // MOE_SHAPE_H

MOE_KERNELS_NS_END
