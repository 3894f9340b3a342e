// moe_jit.h -- run-time compilation of the MoE kernels for one layer shape (moe_jit.cpp).  Private
// to the library.
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "moe_launch.h"

namespace moe {

struct JitResult {
    hipModule_t module;   // owns the kernels below
    JitKernels kernels;
    double compile_ms;    // 0 when the code object came from the cache
    bool from_cache;
    char path[512];       // the code object's file in the cache
};

// Directory of the code-object cache: MOE_JIT_CACHE_DIR, else $XDG_CACHE_HOME/mxfp4_expert_gemv_amd,
// else $HOME/.cache/mxfp4_expert_gemv_amd, else /tmp/mxfp4_expert_gemv_amd_cache.
std::string jit_cache_dir();
// Compiles (or loads from the cache) the kernels of every token count 1..max_tokens for this shape
// on the current device; on failure returns an error status with the message in moe_last_error().
moe_status jit_build(const Shape& sh, int max_tokens, bool normalize, bool mfma, JitResult* out);
void jit_release(JitResult* r);

}  // namespace moe
