// moe_persistent.h -- host interface of the persistent whole-stack kernel (moe_persistent.hip).
// Private to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_launch.h"

namespace moe {
namespace pk {

// Arguments of one stack pass.  Exchange buffers and control words live in the handle's
// workspace and start cleared; every weight tensor is in its canonical row-major layout.
struct StackArgs {
    const LayerPtrs* layers;  // device array [L]
    const uint16_t* x_in;     // [T][H] bf16
    uint64_t* xw;             // [2][kMaxTokens][H/2]   {bf16 x[2i], bf16 x[2i+1] | stamp}
    uint64_t* lw;             // [2][kMaxTokens][E]     {fp32 logit | stamp}
    uint64_t* shw;            // [2][kMaxTokens][I]     {fp32 shared-expert h | stamp}
    uint64_t* hw;             // [2][kMaxSlots][kMaxTokens][I]  {fp32 routed h | stamp}
    uint64_t* dw;             // [2][kMaxSlots][kMaxTokens][H]  {fp32 routed down output | stamp}
    uint32_t* ctl;            // [0] epoch, [1] arrivals, [2] abort, [3] failed round, [4] layer, [5] workgroup
    uint16_t* x_out;          // [T][H] or null
    float* y;                 // [T][H] or null
    int32_t* ids_out;         // [L][T][k] or null
    float* w_out;             // [L][T][k] or null
    uint16_t* trace;          // [L][T][H] or null
    float* x_scale;           // [L][T] or null
    uint8_t* x_codes;         // [L][T][H] or null
    int H, E, k, S, I, L, normalize, rmax;
    long long timeout;        // wall-clock ticks allowed per wait
};

constexpr int kThreads = 512;

// workgroups of a pass: one per compute unit, at most E, H/2 and I*k (so that every workgroup
// owns router rows, hidden rows and SwiGLU outputs)
int grid_size(const Shape& sh, int cus);
int rows_max(const Shape& sh, int n);  // hidden rows owned by one workgroup, at most
size_t lds_bytes(const Shape& sh, int T, int rmax);
hipError_t check_resident(const Shape& sh, int T, int n, int* max_per_cu);
hipError_t launch_stack(const Shape& sh, int T, int n, const StackArgs& args, hipStream_t stream);

// byte sizes of the exchange buffers
inline size_t xw_bytes(const Shape& sh) { return (size_t)2 * kMaxTokens * (sh.H / 2) * 8; }
inline size_t lw_bytes(const Shape& sh) { return (size_t)2 * kMaxTokens * sh.E * 8; }
inline size_t shw_bytes(const Shape& sh) { return (size_t)2 * kMaxTokens * sh.I * 8; }
inline size_t hw_bytes(const Shape& sh) { return (size_t)2 * kMaxSlots * kMaxTokens * sh.I * 8; }
inline size_t dw_bytes(const Shape& sh) { return (size_t)2 * kMaxSlots * kMaxTokens * sh.H * 8; }
constexpr size_t kCtlBytes = 256;

}  // namespace pk
}  // namespace moe
