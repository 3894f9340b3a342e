// head_api.cpp -- C ABI of the FP8 LM head (declarations and contracts in include/moe_decode.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>

#include "moe_launch.h"

namespace head {
hipError_t launch_repack_head(const void* w, const void* s, void* dw, void* ds, int V, int H, bool fp8,
                              hipStream_t stream);
hipError_t launch_quantize_rows(const void* w, bool bf16, int V, int H, void* codes, float* scales,
                                hipStream_t stream);
hipError_t launch_head(const void* w, const float* scale, const uint16_t* x, int T, float* logits, int32_t* argmax,
                       float* pval, int32_t* pidx, unsigned* ticket, const int32_t* draft, int32_t* accept, int V,
                       int H, bool fp8, hipStream_t stream);
hipError_t noalloc_scratch(void** out);
hipError_t launch_head_rowmajor(const void* w, const float* scale, const uint16_t* x, int T, float* logits,
                                int32_t* argmax, void* scratch_dev, int V, int H, hipStream_t stream);
}

namespace probe {
hipError_t launch_stream_read(const void* src, uint64_t bytes, uint32_t* out, int grid, hipStream_t stream);
}

extern "C" moe_status moe_probe_stream_read(const void* src, uint64_t bytes, uint32_t* out, int32_t grid,
                                            void* stream) {
    if (!src || (uintptr_t)src % 16 || bytes % 16 || bytes == 0)
        return moe_fail(MOE_ERR_INVALID_ARG, "src must be 16-byte aligned and bytes a positive multiple of 16");
    if (!out || grid < 1 || grid > 65536) return moe_fail(MOE_ERR_INVALID_ARG, "out is NULL or grid out of range");
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return moe_fail(MOE_ERR_NO_DEVICE, "no HIP device visible");
    }
    hipError_t e = probe::launch_stream_read(src, bytes, out, grid, (hipStream_t)stream);
    if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, "probe launch failed: %s", hipGetErrorString(e));
    return MOE_OK;
}

struct fp8_head_handle {
    int V, H, VT, device;
    bool fp8;          // E4M3 rows with scales, or bf16 rows (bf16_head_create)
    uint8_t* mem;      // repacked weights | scales | per-tile partials | ticket
    void* w;
    float* scale;
    float* pval;
    int32_t* pidx;
    unsigned* ticket;
};

static uint64_t a256(uint64_t v) { return (v + 255) & ~(uint64_t)255; }

static moe_status head_create(int32_t vocab, int32_t hidden, const void* w, const void* row_scale, bool fp8,
                              void* stream, fp8_head_handle** out) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return moe_fail(MOE_ERR_NO_DEVICE, "no HIP device visible");
    }
    fp8_head_handle* h = new (std::nothrow) fp8_head_handle();
    if (!h) return moe_fail(MOE_ERR_OOM, "host allocation failed");
    h->V = vocab;
    h->H = hidden;
    h->VT = (vocab + 63) / 64;
    h->fp8 = fp8;
    (void)hipGetDevice(&h->device);
    const uint64_t wb = a256((uint64_t)h->VT * 64 * hidden * (fp8 ? 1 : 2)), sb = a256((uint64_t)h->VT * 64 * 4);
    const uint64_t pb = a256((uint64_t)h->VT * 4 * 4);
    if (hipMalloc(&h->mem, wb + sb + 2 * pb + 256) != hipSuccess) {
        (void)hipGetLastError();
        delete h;
        return moe_fail(MOE_ERR_OOM, "hipMalloc for the LM head failed");
    }
    h->w = h->mem;
    h->scale = (float*)(h->mem + wb);
    h->pval = (float*)(h->mem + wb + sb);
    h->pidx = (int32_t*)(h->mem + wb + sb + pb);
    h->ticket = (unsigned*)(h->mem + wb + sb + 2 * pb);
    hipError_t e = hipMemsetAsync(h->ticket, 0, 256, (hipStream_t)stream);
    if (e == hipSuccess)
        e = head::launch_repack_head(w, row_scale, h->w, h->scale, vocab, hidden, fp8, (hipStream_t)stream);
    if (e != hipSuccess) {
        (void)hipFree(h->mem);
        delete h;
        return moe_fail(MOE_ERR_HIP, "LM-head repack failed: %s", hipGetErrorString(e));
    }
    *out = h;
    return MOE_OK;
}

static moe_status head_shape_check(int32_t vocab, int32_t hidden, fp8_head_handle** out) {
    if (!out) return moe_fail(MOE_ERR_INVALID_ARG, "out is NULL");
    if (vocab <= 0 || hidden <= 0) return moe_fail(MOE_ERR_INVALID_ARG, "vocab and hidden must be positive");
    if (hidden % 256 || hidden > 2560)
        return moe_fail(MOE_ERR_UNSUPPORTED, "hidden %d (multiple of 256 up to 2560 supported)", hidden);
    return MOE_OK;
}

extern "C" moe_status fp8_head_create(int32_t vocab, int32_t hidden, moe_tensor w, moe_tensor row_scale, void* stream,
                                      fp8_head_handle** out) {
    moe_status st = head_shape_check(vocab, hidden, out);
    if (st != MOE_OK) return st;
    if (!w.ptr || (uintptr_t)w.ptr % 16) return moe_fail(MOE_ERR_INVALID_ARG, "w is NULL or not 16-byte aligned");
    if (!row_scale.ptr || (uintptr_t)row_scale.ptr % 4)
        return moe_fail(MOE_ERR_INVALID_ARG, "row_scale is NULL or not 4-byte aligned");
    if (w.dtype != MOE_DT_E4M3) return moe_fail(MOE_ERR_DTYPE, "w: dtype tag %d, expected E4M3 (%d)", w.dtype, MOE_DT_E4M3);
    if (row_scale.dtype != MOE_DT_FP32)
        return moe_fail(MOE_ERR_DTYPE, "row_scale: dtype tag %d, expected FP32 (%d)", row_scale.dtype, MOE_DT_FP32);
    return head_create(vocab, hidden, w.ptr, row_scale.ptr, true, stream, out);
}

extern "C" moe_status bf16_head_create(int32_t vocab, int32_t hidden, moe_tensor w, void* stream,
                                       fp8_head_handle** out) {
    moe_status st = head_shape_check(vocab, hidden, out);
    if (st != MOE_OK) return st;
    if (!w.ptr || (uintptr_t)w.ptr % 16) return moe_fail(MOE_ERR_INVALID_ARG, "w is NULL or not 16-byte aligned");
    if (w.dtype != MOE_DT_BF16) return moe_fail(MOE_ERR_DTYPE, "w: dtype tag %d, expected BF16 (%d)", w.dtype, MOE_DT_BF16);
    return head_create(vocab, hidden, w.ptr, nullptr, false, stream, out);
}

extern "C" moe_status fp8_head_run(fp8_head_handle* h, const void* x, int32_t T, float* logits, int32_t* argmax,
                                   void* stream) {
    if (!h) return moe_fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (!x || (uintptr_t)x % 16) return moe_fail(MOE_ERR_INVALID_ARG, "x is NULL or not 16-byte aligned");
    if (!argmax) return moe_fail(MOE_ERR_INVALID_ARG, "argmax is NULL");
    if (T < 1 || T > 4) return moe_fail(MOE_ERR_INVALID_ARG, "num_tokens %d out of range [1, 4]", T);
    if (hipSetDevice(h->device) != hipSuccess) return moe_fail(MOE_ERR_HIP, "hipSetDevice failed");
    hipError_t e = head::launch_head(h->w, h->scale, (const uint16_t*)x, T, logits, argmax, h->pval, h->pidx, h->ticket,
                                     nullptr, nullptr, h->V, h->H, h->fp8, (hipStream_t)stream);
    if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, "LM-head launch failed: %s", hipGetErrorString(e));
    return MOE_OK;
}

extern "C" moe_status fp8_head_verify(fp8_head_handle* h, const void* x, int32_t T, const int32_t* draft,
                                      int32_t* argmax, int32_t* accept, void* stream) {
    if (!h) return moe_fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (!x || (uintptr_t)x % 16) return moe_fail(MOE_ERR_INVALID_ARG, "x is NULL or not 16-byte aligned");
    if (!draft || !argmax || !accept) return moe_fail(MOE_ERR_INVALID_ARG, "draft, argmax and accept are required");
    if (T < 2 || T > 4) return moe_fail(MOE_ERR_INVALID_ARG, "num_tokens %d out of range [2, 4]", T);
    if (hipSetDevice(h->device) != hipSuccess) return moe_fail(MOE_ERR_HIP, "hipSetDevice failed");
    hipError_t e = head::launch_head(h->w, h->scale, (const uint16_t*)x, T, nullptr, argmax, h->pval, h->pidx, h->ticket,
                                     draft, accept, h->V, h->H, h->fp8, (hipStream_t)stream);
    if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, "LM-head launch failed: %s", hipGetErrorString(e));
    return MOE_OK;
}

extern "C" moe_status fp8_head_quantize(int32_t rows, int32_t cols, moe_tensor w, void* codes, float* scales,
                                        void* stream) {
    if (rows <= 0 || cols <= 0) return moe_fail(MOE_ERR_INVALID_ARG, "rows and cols must be positive");
    if (cols % 256 || cols > 2560)
        return moe_fail(MOE_ERR_UNSUPPORTED, "cols %d (multiple of 256 up to 2560 supported)", cols);
    if (!w.ptr || (uintptr_t)w.ptr % 16) return moe_fail(MOE_ERR_INVALID_ARG, "w is NULL or not 16-byte aligned");
    if (w.dtype != MOE_DT_BF16 && w.dtype != MOE_DT_FP32)
        return moe_fail(MOE_ERR_DTYPE, "w: dtype tag %d, expected BF16 (%d) or FP32 (%d)", w.dtype, MOE_DT_BF16,
                        MOE_DT_FP32);
    if (!codes || (uintptr_t)codes % 8) return moe_fail(MOE_ERR_INVALID_ARG, "codes is NULL or not 8-byte aligned");
    if (!scales || (uintptr_t)scales % 4) return moe_fail(MOE_ERR_INVALID_ARG, "scales is NULL or not 4-byte aligned");
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return moe_fail(MOE_ERR_NO_DEVICE, "no HIP device visible");
    }
    hipError_t e = head::launch_quantize_rows(w.ptr, w.dtype == MOE_DT_BF16, rows, cols, codes, scales,
                                              (hipStream_t)stream);
    if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, "LM-head quantisation launch failed: %s", hipGetErrorString(e));
    return MOE_OK;
}

extern "C" moe_status fp8_head_run_noalloc(int32_t vocab, int32_t hidden, moe_tensor w, moe_tensor row_scale,
                                           const void* x, int32_t T, float* logits, int32_t* argmax, void* stream) {
    if (vocab <= 0 || hidden <= 0) return moe_fail(MOE_ERR_INVALID_ARG, "vocab and hidden must be positive");
    if (vocab > MOE_NOALLOC_MAX_VOCAB)
        return moe_fail(MOE_ERR_INVALID_ARG, "vocab %d exceeds the no-allocation limit of %d rows", vocab,
                        MOE_NOALLOC_MAX_VOCAB);
    if (hidden % 256 || hidden > 2560)
        return moe_fail(MOE_ERR_UNSUPPORTED, "hidden %d (multiple of 256 up to 2560 supported)", hidden);
    if (!w.ptr || (uintptr_t)w.ptr % 16) return moe_fail(MOE_ERR_INVALID_ARG, "w is NULL or not 16-byte aligned");
    if (!row_scale.ptr || (uintptr_t)row_scale.ptr % 4)
        return moe_fail(MOE_ERR_INVALID_ARG, "row_scale is NULL or not 4-byte aligned");
    if (w.dtype != MOE_DT_E4M3) return moe_fail(MOE_ERR_DTYPE, "w: dtype tag %d, expected E4M3 (%d)", w.dtype, MOE_DT_E4M3);
    if (row_scale.dtype != MOE_DT_FP32)
        return moe_fail(MOE_ERR_DTYPE, "row_scale: dtype tag %d, expected FP32 (%d)", row_scale.dtype, MOE_DT_FP32);
    if (!x || (uintptr_t)x % 16) return moe_fail(MOE_ERR_INVALID_ARG, "x is NULL or not 16-byte aligned");
    if (!argmax) return moe_fail(MOE_ERR_INVALID_ARG, "argmax is NULL");
    if (T < 1 || T > 4) return moe_fail(MOE_ERR_INVALID_ARG, "num_tokens %d out of range [1, 4]", T);
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return moe_fail(MOE_ERR_NO_DEVICE, "no HIP device visible");
    }
    void* sp = nullptr;
    hipError_t e = head::noalloc_scratch(&sp);
    if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, "scratch lookup failed: %s", hipGetErrorString(e));
    e = head::launch_head_rowmajor(w.ptr, (const float*)row_scale.ptr, (const uint16_t*)x, T, logits, argmax, sp, vocab,
                                   hidden, (hipStream_t)stream);
    if (e != hipSuccess) return moe_fail(MOE_ERR_HIP, "LM-head launch failed: %s", hipGetErrorString(e));
    return MOE_OK;
}

extern "C" moe_status fp8_head_destroy(fp8_head_handle* h) {
    if (!h) return MOE_OK;
    (void)hipSetDevice(h->device);
    (void)hipDeviceSynchronize();
    (void)hipFree(h->mem);
    delete h;
    return MOE_OK;
}
