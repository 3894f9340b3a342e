// moe_launch.h -- host-side launcher interface between the C ABI (moe_api.cpp) and the kernels
// (moe_kernels.hip).  Private to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "moe_layout.h"

namespace moe {

struct LayerPtrs {
    const void *router, *w13, *w13s, *w2, *w2s;  // repacked tensors of one layer
    bool w13_mfma;                               // w13 / w13s in the scaled-MFMA operand layout
};

struct RunPtrs {
    const uint16_t* x;  // layer input residual x_l, bf16 [T][H]
    uint16_t* xnext;    // bf16(x_l + y) or null
    float* y;           // fp32 [T][H] or null
    int32_t* ids;       // [T][k] or null
    float* w;           // [T][k] or null
    uint16_t* trace;    // copy of x_l or null
    float* x_scale;     // [T] or null
    uint8_t* x_codes;   // [T][H] or null
    // workspace
    uint8_t* xq;        // 3-4 tokens: [T][H] FP8 codes of the MoE input
    float* xs;          // 3-4 tokens: [T] their scales
    float* logits;      // [T][E]
    unsigned* ticket;   // router arrivals when it takes the top-k (zero between layers)
    SlotTable* slots;
    float* h;           // [T*(k+S)][I]
    float* hamax;       // [T*(k+S)][I/16]
    uint16_t* xn;       // [T][H] MoE input (bf16)
    // 3-4 tokens: the FP8 codes of every h row, computed once per layer
    uint8_t* hq;        // [T*(k+S)][I] FP8 codes of h
    float* hs;          // [T*(k+S)] their scales
    // timing record (graph replays): per kernel kind, the launch's [grid][2] start/end stamps, or null
    unsigned long long* stamp[5];
};

// The kernels one layer launches, by kind; names of their instances for a shape and token count.
enum { kKernInput = 0, kKernRouter, kKernGateup, kKernRequant, kKernDown, kLayerKernels };

// Kernels compiled at run time for one layer shape (MOE_F_JIT): the module function of every kernel
// a layer launches, per token count (fn[T - 1][kind]); kinds a token count does not launch are null.
static_assert(kLayerKernels == 5, "RunPtrs::stamp has one entry per kernel kind");
struct JitKernels {
    hipFunction_t fn[kMaxTokens][kLayerKernels];
};

hipError_t launch_repack(const Shape& sh, const void* router, const void* w13, const void* w13s, const void* w2,
                         const void* w2s, void* d_router, void* d_w13, void* d_w13s, void* d_w2, void* d_w2s,
                         bool mfma, hipStream_t stream);
// ev (nullable) = 4 events recorded before the router and after each of the three kernels.
// jit: run-time compiled kernels to launch instead of the ahead-of-time ones, or null.
hipError_t launch_layer(const Shape& sh, int T, const LayerPtrs& L, const RunPtrs& P, bool normalize,
                        hipStream_t stream, hipEvent_t* ev, const JitKernels* jit);
// Workgroups of the kernel of this kind that a layer launches at T tokens (0 if it launches none).
int layer_grid(const Shape& sh, int T, int kind);
hipError_t launch_clear_u64(unsigned long long* p, uint64_t n, hipStream_t stream);
// Name expressions of the kernel instances a layer of this shape launches at T tokens ("" for kinds
// it does not launch); false for an unsupported shape or token count.
bool jit_kernel_names(const Shape& sh, int T, bool mfma, std::string (&names)[kLayerKernels]);
bool shape_supported(const Shape& sh);

// The same layer launcher built with one layer shape folded in at compile time
// (moe_kernels_flash.hip): for shapes where shape_matches holds.
namespace flash {
bool shape_matches(const Shape& sh);
hipError_t launch_layer(const Shape& sh, int T, const LayerPtrs& L, const RunPtrs& P, bool normalize,
                        hipStream_t stream, hipEvent_t* ev, const JitKernels* jit);
}  // namespace flash

}  // namespace moe

// Records a message for moe_last_error() and returns s (defined in moe_api.cpp).
#include "../../include/moe_decode.h"
moe_status moe_fail(moe_status s, const char* fmt, ...);
