// synth_device.hip -- device twin of the integer part of synth_host.c.
//
// Fills MXFP4 code and scale tensors directly in HBM, so the 42-layer, ~67 GB weight stack never
// crosses PCIe.  Every byte equals what synth_codes / synth_scales write on the host for the
// same (seed, layer, tensor, expert, attempt, index); the generator definition is in
// synth_host.c.  Holds no MoE arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t fmix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

__device__ __forceinline__ uint64_t sm(uint64_t s, uint64_t i) {
    return fmix64(s + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

__device__ __forceinline__ uint64_t key_of(uint64_t seed, uint32_t layer, uint32_t tensor,
                                           uint32_t expert, uint32_t attempt) {
    return sm(sm(sm(sm(seed, layer), tensor), expert), attempt);
}

// One thread writes 8 code bytes (one hash).  bytes_per_expert is a multiple of 8.
__global__ void fill_codes(uint64_t* __restrict__ out, uint64_t words_per_expert, uint32_t n_experts,
                           uint32_t expert0, uint64_t seed, uint32_t layer, uint32_t tensor,
                           uint32_t attempt) {
    const uint64_t total = words_per_expert * n_experts;
    for (uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (uint64_t)gridDim.x * blockDim.x) {
        uint32_t e = (uint32_t)(g / words_per_expert);
        uint64_t w = g - (uint64_t)e * words_per_expert;
        uint64_t key = key_of(seed, layer, tensor, expert0 + e, attempt);
        out[g] = sm(key, w);
    }
}

// One thread writes 4 scale bytes.  bytes_per_expert is a multiple of 4.
__global__ void fill_scales(uint32_t* __restrict__ out, uint64_t dwords_per_expert, uint32_t n_experts,
                            uint32_t expert0, uint64_t seed, uint32_t layer, uint32_t tensor,
                            uint32_t attempt) {
    const uint64_t total = dwords_per_expert * n_experts;
    for (uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (uint64_t)gridDim.x * blockDim.x) {
        uint32_t e = (uint32_t)(g / dwords_per_expert);
        uint64_t d = g - (uint64_t)e * dwords_per_expert;
        uint64_t key = key_of(seed, layer, tensor, expert0 + e, attempt);
        uint32_t v = 0;
        for (int b = 0; b < 4; ++b) v |= (uint32_t)(121 + sm(key, 4 * d + b) % 5) << (8 * b);
        out[g] = v;
    }
}

}  // namespace

extern "C" {

// Returns 0 on success, a hipError_t value otherwise, -1 on bad arguments.
int synth_dev_codes(void* dst, uint64_t bytes_per_expert, uint32_t n_experts, uint32_t expert0,
                    uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t attempt, hipStream_t stream) {
    if (!dst || bytes_per_expert % 8 || ((uintptr_t)dst & 7)) return -1;
    uint64_t total = bytes_per_expert / 8 * n_experts;
    if (total == 0) return 0;
    uint64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_codes, dim3((unsigned)blocks), dim3(256), 0, stream, (uint64_t*)dst,
                       bytes_per_expert / 8, n_experts, expert0, seed, layer, tensor, attempt);
    return (int)hipGetLastError();
}

int synth_dev_scales(void* dst, uint64_t bytes_per_expert, uint32_t n_experts, uint32_t expert0,
                     uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t attempt, hipStream_t stream) {
    if (!dst || bytes_per_expert % 4 || ((uintptr_t)dst & 3)) return -1;
    uint64_t total = bytes_per_expert / 4 * n_experts;
    if (total == 0) return 0;
    uint64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_scales, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t*)dst,
                       bytes_per_expert / 4, n_experts, expert0, seed, layer, tensor, attempt);
    return (int)hipGetLastError();
}

}  // extern "C"
