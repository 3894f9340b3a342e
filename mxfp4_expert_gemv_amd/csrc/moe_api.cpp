// moe_api.cpp -- C ABI of the MI355X MoE decode library (declarations and contracts in
// include/moe_decode.h).  Validation runs before any HIP call; every unsupported request is an
// error, never a fallback to a slower path.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "../../include/moe_decode.h"
#include "moe_jit.h"
#include "moe_launch.h"


using moe::Shape;

static thread_local char g_err[512];

moe_status moe_fail(moe_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

#define fail moe_fail

static uint64_t align256(uint64_t v) { return (v + 255) & ~(uint64_t)255; }

struct moe_decode_handle {
    moe_decode_config cfg;
    Shape sh;
    int device;
    // per layer: one allocation holding router, w13, w13_s, w2, w2_s (256-byte aligned pieces)
    std::vector<uint8_t*> layer_mem;
    std::vector<char> layer_set;
    uint64_t off_w13, off_w13s, off_w2, off_w2s, layer_bytes;
    // workspace
    uint8_t* ws;
    uint64_t ws_bytes;
    uint8_t* xq;
    float* xs;
    uint16_t* xbuf[2];
    float* logits;
    unsigned* ticket;
    moe::SlotTable* slots;
    float* h;
    float* hamax;
    uint16_t* xn;
    uint8_t* hq;
    float* hs;
    // captured launch sequences of whole runs, keyed by their arguments
    struct GraphEntry {
        const void* x;
        int32_t T;
        moe_outputs out;
        bool stamped;  // the timing record's variant (mode 1)
        hipGraphExec_t exec;
    };
    std::vector<GraphEntry> graphs;
    hipStream_t capture_stream = nullptr;
    // timing instrumentation.  Mode 0: two events around each kernel of each layer of each recorded
    // run (kernels launched one by one).  Mode 1: graph replays whose kernels write wall-clock stamps
    // per workgroup into `stamps` (offsets per layer and kernel kind), reduced after each run.
    int timing_mode = 0;
    std::vector<hipEvent_t> events;
    std::vector<int> timing_T;  // token count of each recorded run
    int timing_max_runs = 0, timing_runs = 0;
    unsigned long long* stamps = nullptr;
    uint64_t stamp_count = 0;                          // 64-bit words
    std::vector<uint64_t> stamp_off;                   // [L][kinds] word offsets
    std::vector<unsigned long long> stamp_host;
    double clock_khz = 0.0;
    double span_ms[MOE_TIMING_CLASSES] = {}, gap_ms[MOE_TIMING_CLASSES] = {};
    uint64_t span_n[MOE_TIMING_CLASSES] = {}, gap_n[MOE_TIMING_CLASSES] = {};
    // kernels compiled at run time for this shape (MOE_F_JIT)
    bool jit_on = false;
    // the ahead-of-time build with this shape folded in (moe::flash), unless MOE_F_GENERIC
    bool flash = false;
    moe::JitResult jit{};
};

// Frees the timing record; queued runs may still record its events or write its stamps, so the
// device is drained first.
static void free_events(moe_decode_handle* h) {
    if (!h->events.empty() || h->stamps) (void)hipDeviceSynchronize();
    for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
    h->events.clear();
    h->timing_T.clear();
    h->timing_max_runs = h->timing_runs = 0;
    if (h->stamps) (void)hipFree(h->stamps);
    h->stamps = nullptr;
    h->stamp_count = 0;
    for (int c = 0; c < MOE_TIMING_CLASSES; ++c) {
        h->span_ms[c] = h->gap_ms[c] = 0.0;
        h->span_n[c] = h->gap_n[c] = 0;
    }
}

extern "C" const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape";
        case MOE_ERR_DTYPE: return "dtype tag mismatch";
        case MOE_ERR_OOM: return "out of device memory";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_NO_DEVICE: return "no HIP device";
        case MOE_ERR_STATE: return "invalid state";
    }
    return "unknown status";
}

extern "C" const char* moe_last_error(void) { return g_err; }

static moe_status check_config(const moe_decode_config* c) {
    if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
    if (c->struct_size != sizeof(moe_decode_config))
        return fail(MOE_ERR_INVALID_ARG, "config struct_size %u != %zu", c->struct_size, sizeof(moe_decode_config));
    if (c->hidden <= 0 || c->num_experts <= 0 || c->top_k <= 0 || c->inter <= 0 || c->max_tokens <= 0 ||
        c->num_layers <= 0 || c->num_shared < 0)
        return fail(MOE_ERR_INVALID_ARG, "sizes must be positive");
    if (c->top_k > c->num_experts) return fail(MOE_ERR_INVALID_ARG, "top_k %d > num_experts %d", c->top_k, c->num_experts);
    if (c->num_shared > 1) return fail(MOE_ERR_UNSUPPORTED, "num_shared %d (0 or 1 supported)", c->num_shared);
    if (c->hidden % 256 || c->hidden > 2560)
        return fail(MOE_ERR_UNSUPPORTED, "hidden %d (multiple of 256 up to 2560 supported)", c->hidden);
    if (c->num_experts > 512 || c->num_experts % 8)
        return fail(MOE_ERR_UNSUPPORTED, "num_experts %d (multiple of 8 up to 512 supported)", c->num_experts);
    if (c->top_k > moe::kMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "top_k %d > 8", c->top_k);
    if (c->max_tokens > moe::kMaxTokens) return fail(MOE_ERR_UNSUPPORTED, "max_tokens %d > 4", c->max_tokens);
    const moe::Shape sh{c->hidden, c->num_experts, c->top_k, c->num_shared, c->inter};
    if (c->inter % moe::kBlock || !moe::shape_supported(sh))
        return fail(MOE_ERR_UNSUPPORTED, "hidden %d / inter %d: no kernel for this shape (inter 64, 128, 256 or 768)",
                    c->hidden, c->inter);
    if (c->flags & ~(uint32_t)(MOE_F_RMSNORM_INPUT | MOE_F_DIRECT_LAUNCH | MOE_F_JIT | MOE_F_MFMA | MOE_F_GENERIC))
        return fail(MOE_ERR_INVALID_ARG, "unknown flags 0x%x", c->flags);
    return MOE_OK;
}

static moe_status device_present() {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return fail(MOE_ERR_NO_DEVICE, "no HIP device visible");
    }
    return MOE_OK;
}

// Destroys the captured graphs.  run only enqueues, so launches of them may still be executing on
// the callers' streams: the device is drained first (this happens when the 16 entries are full, on
// timing changes and at destroy, not on the replay path).
static void free_graphs(moe_decode_handle* h) {
    if (h->graphs.empty()) return;
    (void)hipDeviceSynchronize();
    for (auto& g : h->graphs) (void)hipGraphExecDestroy(g.exec);
    h->graphs.clear();
}

static void free_handle(moe_decode_handle* h) {
    free_events(h);
    moe::jit_release(&h->jit);
    free_graphs(h);
    if (h->capture_stream) (void)hipStreamDestroy(h->capture_stream);
    for (uint8_t* p : h->layer_mem)
        if (p) (void)hipFree(p);
    if (h->ws) (void)hipFree(h->ws);
    delete h;
}

extern "C" moe_status moe_decode_create(const moe_decode_config* cfg, void* stream, moe_decode_handle** out) {
    moe_status s = check_config(cfg);
    if (s != MOE_OK) return s;
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    if ((s = device_present()) != MOE_OK) return s;
    (void)stream;
    moe_decode_handle* h = new (std::nothrow) moe_decode_handle();
    if (!h) return fail(MOE_ERR_OOM, "host allocation failed");
    h->cfg = *cfg;
    h->sh = Shape{cfg->hidden, cfg->num_experts, cfg->top_k, cfg->num_shared, cfg->inter};
    const Shape& sh = h->sh;
    if (hipGetDevice(&h->device) != hipSuccess) {
        delete h;
        return fail(MOE_ERR_HIP, "hipGetDevice failed");
    }
    const uint64_t nexp = (uint64_t)sh.E + sh.S;
    h->off_w13 = align256(sh.router_bytes());
    h->off_w13s = h->off_w13 + align256(nexp * sh.w13_bytes_per_expert());
    h->off_w2 = h->off_w13s + align256(nexp * sh.w13s_bytes_per_expert());
    h->off_w2s = h->off_w2 + align256(nexp * sh.w2_bytes_per_expert());
    h->layer_bytes = h->off_w2s + align256(nexp * sh.w2s_bytes_per_expert());
    h->layer_mem.assign(cfg->num_layers, nullptr);
    h->layer_set.assign(cfg->num_layers, 0);
    for (int l = 0; l < cfg->num_layers; ++l) {
        if (hipMalloc(&h->layer_mem[l], h->layer_bytes) != hipSuccess) {
            (void)hipGetLastError();
            free_handle(h);
            return fail(MOE_ERR_OOM, "hipMalloc of %llu bytes for layer %d failed", (unsigned long long)h->layer_bytes, l);
        }
    }
    // workspace
    const int T = moe::kMaxTokens;
    uint64_t o = 0;
    const uint64_t o_xq = o; o += align256((uint64_t)T * sh.H);
    const uint64_t o_xs = o; o += 256;
    const uint64_t o_xb0 = o; o += align256((uint64_t)T * sh.H * 2);
    const uint64_t o_xb1 = o; o += align256((uint64_t)T * sh.H * 2);
    const uint64_t o_lg = o; o += align256((uint64_t)T * sh.E * 4);
    const uint64_t o_tk = o; o += 256;
    const uint64_t o_slot = o; o += align256(sizeof(moe::SlotTable));
    const uint64_t o_h = o; o += align256((uint64_t)sh.pairs(T) * sh.I * 4);
    const uint64_t o_ham = o; o += align256((uint64_t)sh.pairs(T) * sh.gu_tiles() * 4);
    const uint64_t o_xn = o; o += align256((uint64_t)T * sh.H * 2);
    const uint64_t o_hq = o; o += align256((uint64_t)sh.pairs(T) * sh.I);
    const uint64_t o_hs = o; o += align256((uint64_t)sh.pairs(T) * 4);
    h->ws_bytes = o;
    if (hipMalloc(&h->ws, o) != hipSuccess) {
        (void)hipGetLastError();
        free_handle(h);
        return fail(MOE_ERR_OOM, "workspace hipMalloc failed");
    }
    if (hipMemset(h->ws, 0, o) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        free_handle(h);
        return fail(MOE_ERR_HIP, "workspace clear failed");
    }
    if (hipStreamCreateWithFlags(&h->capture_stream, hipStreamNonBlocking) != hipSuccess) {
        free_handle(h);
        return fail(MOE_ERR_HIP, "hipStreamCreate failed");
    }
    h->xq = h->ws + o_xq;
    h->xs = (float*)(h->ws + o_xs);
    h->xbuf[0] = (uint16_t*)(h->ws + o_xb0);
    h->xbuf[1] = (uint16_t*)(h->ws + o_xb1);
    h->logits = (float*)(h->ws + o_lg);
    h->ticket = (unsigned*)(h->ws + o_tk);
    h->slots = (moe::SlotTable*)(h->ws + o_slot);
    h->h = (float*)(h->ws + o_h);
    h->hamax = (float*)(h->ws + o_ham);
    h->xn = (uint16_t*)(h->ws + o_xn);
    h->hq = h->ws + o_hq;
    h->hs = (float*)(h->ws + o_hs);
    if (cfg->flags & MOE_F_JIT) {
        s = moe::jit_build(sh, cfg->max_tokens, (cfg->flags & MOE_F_RMSNORM_INPUT) != 0,
                           (cfg->flags & MOE_F_MFMA) != 0, &h->jit);
        if (s != MOE_OK) {
            free_handle(h);
            return s;
        }
        h->jit_on = true;
    }
    h->flash = !h->jit_on && !(cfg->flags & MOE_F_GENERIC) && moe::flash::shape_matches(sh);
    *out = h;
    g_err[0] = 0;
    return MOE_OK;
}

static moe_status check_tensor(const moe_tensor& t, moe_dtype want, const char* name) {
    if (!t.ptr) return fail(MOE_ERR_INVALID_ARG, "%s: NULL pointer", name);
    if ((uintptr_t)t.ptr % 16) return fail(MOE_ERR_INVALID_ARG, "%s: pointer not 16-byte aligned", name);
    if (t.dtype != want) return fail(MOE_ERR_DTYPE, "%s: dtype tag %d, expected %d", name, t.dtype, (int)want);
    return MOE_OK;
}

extern "C" moe_status moe_decode_set_layer(moe_decode_handle* h, int32_t layer, const moe_layer_desc* d,
                                           void* stream) {
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (!d) return fail(MOE_ERR_INVALID_ARG, "descriptor is NULL");
    if (layer < 0 || layer >= h->cfg.num_layers)
        return fail(MOE_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, h->cfg.num_layers);
    moe_status s;
    if ((s = check_tensor(d->router, MOE_DT_BF16, "router")) != MOE_OK) return s;
    if ((s = check_tensor(d->w13, MOE_DT_E2M1X2, "w13")) != MOE_OK) return s;
    if ((s = check_tensor(d->w13_s, MOE_DT_E8M0, "w13_s")) != MOE_OK) return s;
    if ((s = check_tensor(d->w2, MOE_DT_E2M1X2, "w2")) != MOE_OK) return s;
    if ((s = check_tensor(d->w2_s, MOE_DT_E8M0, "w2_s")) != MOE_OK) return s;
    if (hipSetDevice(h->device) != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice failed");
    uint8_t* m = h->layer_mem[layer];
    hipError_t e = moe::launch_repack(h->sh, d->router.ptr, d->w13.ptr, d->w13_s.ptr, d->w2.ptr, d->w2_s.ptr, m,
                                      m + h->off_w13, m + h->off_w13s, m + h->off_w2, m + h->off_w2s,
                                      (h->cfg.flags & MOE_F_MFMA) != 0, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "repack launch failed: %s", hipGetErrorString(e));
    h->layer_set[layer] = 1;
    return MOE_OK;
}

// Enqueues the kernels of every layer on `stream` (timing: with the event records; stamped: with the
// wall-clock stamps of the timing record, after clearing them).
static moe_status enqueue_run(moe_decode_handle* h, const void* x, int32_t T, const moe_outputs& o, hipStream_t stream,
                              bool timing, bool stamped = false) {
    if (stamped) {
        hipError_t e = moe::launch_clear_u64(h->stamps, h->stamp_count, stream);
        if (e != hipSuccess) return fail(MOE_ERR_HIP, "timing record clear failed: %s", hipGetErrorString(e));
    }
    const Shape& sh = h->sh;
    const bool norm = (h->cfg.flags & MOE_F_RMSNORM_INPUT) != 0;
    const int L = h->cfg.num_layers;
    const size_t TH = (size_t)T * sh.H;
    for (int l = 0; l < L; ++l) {
        const uint8_t* m = h->layer_mem[l];
        moe::LayerPtrs lp{m, m + h->off_w13, m + h->off_w13s, m + h->off_w2, m + h->off_w2s,
                          (h->cfg.flags & MOE_F_MFMA) != 0};
        moe::RunPtrs p{};
        p.x = l == 0 ? (const uint16_t*)x : h->xbuf[l & 1];
        const bool last = l == L - 1;
        p.xnext = last ? (uint16_t*)o.x_out : h->xbuf[(l + 1) & 1];
        p.y = last ? o.y : nullptr;
        p.ids = o.topk_ids ? o.topk_ids + (size_t)l * T * sh.k : nullptr;
        p.w = o.topk_w ? o.topk_w + (size_t)l * T * sh.k : nullptr;
        p.trace = o.x_trace ? (uint16_t*)o.x_trace + (size_t)l * TH : nullptr;
        p.x_scale = o.x_scale ? o.x_scale + (size_t)l * T : nullptr;
        p.x_codes = o.x_codes ? o.x_codes + (size_t)l * TH : nullptr;
        p.xq = h->xq;
        p.xs = h->xs;
        p.logits = h->logits;
        p.ticket = h->ticket;
        p.slots = h->slots;
        p.h = h->h;
        p.hamax = h->hamax;
        p.xn = h->xn;
        p.hq = h->hq;
        p.hs = h->hs;
        hipEvent_t* ev = nullptr;
        if (timing) ev = &h->events[((size_t)h->timing_runs * L + l) * 2 * MOE_TIMING_CLASSES];
        if (stamped)
            for (int k = 0; k < MOE_TIMING_CLASSES; ++k)
                p.stamp[k] = moe::layer_grid(sh, T, k) ? h->stamps + h->stamp_off[(size_t)l * MOE_TIMING_CLASSES + k]
                                                       : nullptr;
        hipError_t e = h->flash ? moe::flash::launch_layer(sh, T, lp, p, norm, stream, ev, nullptr)
                                : moe::launch_layer(sh, T, lp, p, norm, stream, ev, h->jit_on ? &h->jit.kernels : nullptr);
        if (e != hipSuccess) return fail(MOE_ERR_HIP, "layer %d launch failed: %s", l, hipGetErrorString(e));
    }
    return MOE_OK;
}

// Timing record, mode 1: waits for the pass, reads the stamps and adds, per kernel kind, the span from
// its first workgroup's start to its last workgroup's end, and the gap from the previous kernel's end
// to its start (the first kernel of the pass has no previous one).
static moe_status reduce_stamps(moe_decode_handle* h, int T, hipStream_t stream) {
    if (hipStreamSynchronize(stream) != hipSuccess) return fail(MOE_ERR_HIP, "timing record: synchronisation failed");
    h->stamp_host.resize(h->stamp_count);
    if (hipMemcpy(h->stamp_host.data(), h->stamps, h->stamp_count * 8, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(MOE_ERR_HIP, "timing record: read-back failed");
    const double ms_per_tick = 1.0 / h->clock_khz;
    const int L = h->cfg.num_layers;
    bool have_prev = false;
    unsigned long long prev_end = 0;
    for (int l = 0; l < L; ++l)
        for (int k = 0; k < MOE_TIMING_CLASSES; ++k) {
            const int grid = moe::layer_grid(h->sh, T, k);
            if (!grid) continue;
            const unsigned long long* s = h->stamp_host.data() + h->stamp_off[(size_t)l * MOE_TIMING_CLASSES + k];
            unsigned long long lo = ~0ull, hi = 0;
            for (int b = 0; b < grid; ++b) {
                if (!s[2 * b] || !s[2 * b + 1]) continue;  // a workgroup that wrote no record
                lo = std::min(lo, s[2 * b]);
                hi = std::max(hi, s[2 * b + 1]);
            }
            if (hi == 0) return fail(MOE_ERR_HIP, "timing record: kernel %d of layer %d left no stamps", k, l);
            h->span_ms[k] += (double)(hi - lo) * ms_per_tick;
            h->span_n[k] += 1;
            if (have_prev) {
                h->gap_ms[k] += (double)((long long)lo - (long long)prev_end) * ms_per_tick;
                h->gap_n[k] += 1;
            }
            have_prev = true;
            prev_end = hi;
        }
    ++h->timing_runs;
    return MOE_OK;
}

extern "C" moe_status moe_decode_run(moe_decode_handle* h, const void* x, int32_t T, const moe_outputs* out,
                                     void* stream) {
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (!x || (uintptr_t)x % 16) return fail(MOE_ERR_INVALID_ARG, "x is NULL or not 16-byte aligned");
    if (T < 1 || T > h->cfg.max_tokens)
        return fail(MOE_ERR_INVALID_ARG, "num_tokens %d out of range [1, %d]", T, h->cfg.max_tokens);
    if (out && out->struct_size != sizeof(moe_outputs))
        return fail(MOE_ERR_INVALID_ARG, "outputs struct_size %u != %zu", out->struct_size, sizeof(moe_outputs));
    const int L = h->cfg.num_layers;
    for (int l = 0; l < L; ++l)
        if (!h->layer_set[l]) return fail(MOE_ERR_STATE, "layer %d has not been set", l);
    moe_outputs o{};
    if (out) o = *out;
    if (o.x_out && (uintptr_t)o.x_out % 4) return fail(MOE_ERR_INVALID_ARG, "x_out not 4-byte aligned");
    if (o.x_codes && (uintptr_t)o.x_codes % 8) return fail(MOE_ERR_INVALID_ARG, "x_codes not 8-byte aligned");
    if (hipSetDevice(h->device) != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice failed");
    const bool timing = h->timing_runs < h->timing_max_runs;
    const bool stamped = timing && h->timing_mode == 1;
    if ((timing && !stamped) || (h->cfg.flags & MOE_F_DIRECT_LAUNCH)) {
        moe_status st = enqueue_run(h, x, T, o, (hipStream_t)stream, timing && !stamped, stamped);
        if (st == MOE_OK && timing && !stamped) {
            h->timing_T.push_back(T);
            ++h->timing_runs;
        }
        if (st == MOE_OK && stamped) st = reduce_stamps(h, T, (hipStream_t)stream);
        return st;
    }
    // replay the captured launch sequence of this exact call (capture it on first use)
    for (auto& g : h->graphs) {
        if (g.x == x && g.T == T && g.stamped == stamped && memcmp(&g.out, &o, sizeof o) == 0) {
            if (hipGraphLaunch(g.exec, (hipStream_t)stream) != hipSuccess)
                return fail(MOE_ERR_HIP, "hipGraphLaunch failed");
            return stamped ? reduce_stamps(h, T, (hipStream_t)stream) : MOE_OK;
        }
    }
    if (h->graphs.size() >= 16) free_graphs(h);
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(h->capture_stream, hipStreamCaptureModeThreadLocal) != hipSuccess)
        return fail(MOE_ERR_HIP, "hipStreamBeginCapture failed");
    moe_status st = enqueue_run(h, x, T, o, h->capture_stream, false, stamped);
    hipError_t e = hipStreamEndCapture(h->capture_stream, &graph);
    if (st != MOE_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return st;
    }
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGraphInstantiate failed: %s", hipGetErrorString(e));
    h->graphs.push_back({x, T, o, stamped, exec});
    if (hipGraphLaunch(exec, (hipStream_t)stream) != hipSuccess) return fail(MOE_ERR_HIP, "hipGraphLaunch failed");
    return stamped ? reduce_stamps(h, T, (hipStream_t)stream) : MOE_OK;
}

extern "C" moe_status moe_decode_timing_enable(moe_decode_handle* h, int32_t max_runs, int32_t mode) {
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (max_runs < 0 || max_runs > 100000) return fail(MOE_ERR_INVALID_ARG, "max_runs %d out of range", max_runs);
    if (mode != 0 && mode != 1) return fail(MOE_ERR_INVALID_ARG, "timing mode %d (0 or 1)", mode);
    if (hipSetDevice(h->device) != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice failed");
    free_events(h);
    free_graphs(h);  // a stamped graph holds the record's pointers
    h->timing_mode = mode;
    if (max_runs == 0) return MOE_OK;
    if (mode == 0) {
        const size_t n = (size_t)max_runs * h->cfg.num_layers * 2 * MOE_TIMING_CLASSES;
        h->events.reserve(n);
        for (size_t i = 0; i < n; ++i) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) {
                free_events(h);
                return fail(MOE_ERR_HIP, "hipEventCreate failed");
            }
            h->events.push_back(e);
        }
    } else {
        int khz = 0;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, h->device) != hipSuccess || khz <= 0)
            return fail(MOE_ERR_HIP, "wall clock rate query failed");
        h->clock_khz = khz;
        const int L = h->cfg.num_layers;
        h->stamp_off.assign((size_t)L * MOE_TIMING_CLASSES, 0);
        uint64_t words = 0;
        for (int l = 0; l < L; ++l)
            for (int k = 0; k < MOE_TIMING_CLASSES; ++k) {
                int g = 0;
                for (int T = 1; T <= h->cfg.max_tokens; ++T) g = std::max(g, moe::layer_grid(h->sh, T, k));
                h->stamp_off[(size_t)l * MOE_TIMING_CLASSES + k] = words;
                words += 2 * (uint64_t)g;
            }
        if (hipMalloc(&h->stamps, words * 8) != hipSuccess) {
            (void)hipGetLastError();
            return fail(MOE_ERR_OOM, "timing record allocation failed");
        }
        h->stamp_count = words;
    }
    h->timing_max_runs = max_runs;
    return MOE_OK;
}

extern "C" moe_status moe_decode_timing_read(moe_decode_handle* h, moe_decode_timing* out) {
    if (!h || !out) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
    if (out->struct_size != sizeof(moe_decode_timing))
        return fail(MOE_ERR_INVALID_ARG, "timing struct_size %u != %zu", out->struct_size, sizeof(moe_decode_timing));
    const uint32_t ss = out->struct_size;
    memset(out, 0, sizeof *out);
    out->struct_size = ss;
    out->mode = h->timing_mode;
    out->runs = h->timing_runs;
    const int L = h->cfg.num_layers;
    if (h->timing_mode == 1) {
        for (int c = 0; c < MOE_TIMING_CLASSES; ++c) {
            out->launches[c] = h->span_n[c];
            out->total_ms[c] = h->span_ms[c];
            out->gap_launches[c] = h->gap_n[c];
            out->gap_ms[c] = h->gap_ms[c];
            h->span_ms[c] = h->gap_ms[c] = 0.0;
            h->span_n[c] = h->gap_n[c] = 0;
        }
        h->timing_runs = 0;
        return MOE_OK;
    }
    for (int r = 0; r < h->timing_runs; ++r) {
        const int T = h->timing_T[r];
        for (int l = 0; l < L; ++l) {
            hipEvent_t* ev = &h->events[((size_t)r * L + l) * 2 * MOE_TIMING_CLASSES];
            for (int c = 0; c < MOE_TIMING_CLASSES; ++c) {
                if (!moe::layer_grid(h->sh, T, c)) continue;
                float ms = 0.0f;
                if (hipEventSynchronize(ev[2 * c + 1]) != hipSuccess ||
                    hipEventElapsedTime(&ms, ev[2 * c], ev[2 * c + 1]) != hipSuccess)
                    return fail(MOE_ERR_HIP, "event timing failed");
                out->total_ms[c] += ms;
                out->launches[c] += 1;
            }
        }
    }
    h->timing_runs = 0;
    h->timing_T.clear();
    return MOE_OK;
}

extern "C" moe_status moe_decode_query(const moe_decode_handle* h, moe_decode_info* info) {
    if (!h || !info) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
    if (info->struct_size != sizeof(moe_decode_info))
        return fail(MOE_ERR_INVALID_ARG, "info struct_size %u != %zu", info->struct_size, sizeof(moe_decode_info));
    const Shape& sh = h->sh;
    memset(info->variant, 0, sizeof info->variant);
    snprintf(info->variant, sizeof info->variant, "gfx950-3k-gu%dx%d-dn%dx%d-%s%s%s%s", sh.gw(), sh.bpl(),
             sh.ksub(), sh.iters(), (h->cfg.flags & MOE_F_DIRECT_LAUNCH) ? "direct" : "graph", h->jit_on ? "-jit" : "",
             (h->cfg.flags & MOE_F_MFMA) ? "-mfma" : "", h->flash ? "-flash" : "");
    info->weight_bytes = h->layer_bytes * (uint64_t)h->cfg.num_layers;
    info->workspace_bytes = h->ws_bytes;
    const uint64_t expert = sh.w13_bytes_per_expert() + sh.w13s_bytes_per_expert() + sh.w2_bytes_per_expert() +
                            sh.w2s_bytes_per_expert();
    info->bytes_per_layer_t1 = (uint64_t)sh.E * sh.H * 2 + (uint64_t)(sh.k + sh.S) * expert;
    int n = 0;
    for (char c : h->layer_set) n += c ? 1 : 0;
    info->layers_set = n;
    info->jit_compile_ms = h->jit_on ? h->jit.compile_ms : 0.0;
    info->jit_from_cache = h->jit_on && h->jit.from_cache ? 1 : 0;
    memset(info->jit_code_object, 0, sizeof info->jit_code_object);
    if (h->jit_on) snprintf(info->jit_code_object, sizeof info->jit_code_object, "%s", h->jit.path);
    return MOE_OK;
}

extern "C" moe_status moe_decode_check(moe_decode_handle* h) {
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (hipSetDevice(h->device) != hipSuccess) return fail(MOE_ERR_HIP, "hipSetDevice failed");
    const hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "device synchronisation failed: %s", hipGetErrorString(e));
    return MOE_OK;
}

extern "C" moe_status moe_decode_destroy(moe_decode_handle* h) {
    if (!h) return MOE_OK;
    (void)hipSetDevice(h->device);
    (void)hipDeviceSynchronize();
    free_handle(h);
    return MOE_OK;
}
