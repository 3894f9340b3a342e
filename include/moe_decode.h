/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) W4A8 sparse-MoE decode library.
 *
 * One call of moe_decode_run computes, for T <= 4 tokens, the decode step of a stack of sparse
 * Mixture-of-Experts layers with MXFP4 expert weights and FP8 (E4M3) activations:
 *   router GEMV (bf16) -> top-k over the routed experts -> softmax over the k selected logits ->
 *   per-token FP8 quantisation of the input -> dequant-on-the-fly gate/up GEMVs, h = SiLU(gate)*up ->
 *   per-(token, expert) FP8 requantisation of h -> dequant-on-the-fly down GEMV ->
 *   weighted combine y = sum_r w_r d_(id_r) + d_shared.
 * With several layers each layer's input is an unweighted RMSNorm of the bf16 residual and the
 * residual is updated as x <- bf16(x + y).  fp8_head_* is the companion FP8 LM-head GEMV with a
 * per-token argmax.
 *
 * Passages that define the operation (titles as printed on the pages):
 *   - 8 of 512 routed experts plus one shared expert per MoE layer: tanhow.com, "NVIDIA 在单台 DGX
 *     Spark 上叠加三项优化，Ling-3.0-flash 的 MoE 推理吞吐提升 42.5%", section "Ling 3.0 是什么",
 *     sparse-MoE bullet; aivibenews.ru, "Три приёма ускорить MoE-инференс на DGX Spark без потери
 *     GSM8K", introduction.
 *   - expert layers of width 768, MXFP4 expert kernel: tanhow.com, section "三项优化是什么", item 1;
 *     devotd.net, "dgx-spark-moe-inference-optimizations", section 2 (MXFP4 is a blocked 4-bit float).
 *   - 4-bit weights with 8-bit activations (W4A8): tanhow.com, section "为什么 DGX Spark 上的 MoE
 *     解码是内存受限的"; devotd.net, section 2, last paragraph.
 *   - 4-position verify touching up to 32 experts: tanhow.com, section "三项优化是什么", item 3;
 *     devotd.net, section 3.
 *   - FP8 LM head of 157,184 x 2,560 (hence hidden size 2,560), read in full per token:
 *     tanhow.com, section "三项优化是什么", item 2; devotd.net, section 2.
 *   - the silent FP8-read-as-BF16 fallback and the advice to check at start-up that every
 *     optimisation is active: tanhow.com, section "三项优化是什么", paragraph on the integration
 *     trap; devotd.net, section 3.  Hence every tensor carries a dtype tag that is checked, an
 *     unsupported request is an error (never a slower fallback), and moe_decode_query reports the
 *     kernel variant in use.
 *
 * Formats (OCP MX v1.0 and OCP FP8):
 *   E2M1X2  two E2M1 codes per byte, the even element in the low nibble.
 *   E8M0    one byte per 32 consecutive elements along the reduction (K) dimension, 2^(b-127).
 *   E4M3    OCP "fn" FP8, bias 7, max 448, no infinities.
 *   BF16    bfloat16 bits.
 *
 * Conventions for every function:
 *   - Pointers inside moe_tensor / moe_outputs and the x argument are DEVICE pointers on the
 *     device that was current at create time.  Config and descriptor structs are host memory.
 *   - All arguments are validated before any HIP call; a failure returns an error status and
 *     leaves the handle unchanged.  moe_last_error() gives a message for the last failure of the
 *     calling thread.
 *   - run / set_layer only enqueue work on the given stream (hipStream_t, 0 = default stream) and
 *     return; asynchronous device faults surface at the caller's next synchronisation.
 *   - A handle is used from one stream at a time.  Calls that overlap on one handle race on its
 *     workspace.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* NULL/unaligned pointer, bad size, bad struct_size */
    MOE_ERR_UNSUPPORTED = -2, /* valid shape this build has no kernel for (never a fallback) */
    MOE_ERR_DTYPE = -3,       /* a tensor's dtype tag is not the one the slot requires */
    MOE_ERR_OOM = -4,         /* device allocation failed */
    MOE_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed */
    MOE_ERR_NO_DEVICE = -6,   /* no HIP device visible */
    MOE_ERR_STATE = -7        /* e.g. run before every layer was set */
} moe_status;

typedef enum {
    MOE_DT_BF16 = 1,
    MOE_DT_FP32 = 2,
    MOE_DT_E4M3 = 3,
    MOE_DT_E2M1X2 = 4,
    MOE_DT_E8M0 = 5
} moe_dtype;

/* flags of moe_decode_config */
#define MOE_F_RMSNORM_INPUT 0x1u /* each layer's MoE input is RMSNorm(x), eps 1e-6, unweighted */
#define MOE_F_DIRECT_LAUNCH 0x2u /* launch the kernels on the stream at every run instead of replaying
                                    a HIP graph captured on the first run with the same arguments */
#define MOE_F_JIT 0x8u           /* compile the kernels at create time, with hipRTC, for this shape (H, E, k,
                                    S, I), input normalisation and the current device's architecture,
                                    instead of using the ahead-of-time build (tanhow.com, "NVIDIA 在单台 DGX
                                    Spark 上叠加三项优化...", section "三项优化是什么", item 1: kernels compiled
                                    at run time for the actual shapes, dtypes and GPU).  The code object is
                                    cached on disk (MOE_JIT_CACHE_DIR, else $XDG_CACHE_HOME or
                                    $HOME/.cache under mxfp4_expert_gemv_amd), keyed by shape, architecture
                                    and a digest of source, options and kernels; a later create with the
                                    same key loads it.  A failed compile makes create fail (MOE_ERR_HIP);
                                    nothing falls back to the ahead-of-time kernels. */
#define MOE_F_MFMA 0x10u         /* gate/up dot products on the matrix cores: per MX block (32 K) one
                                    v_mfma_f32_16x16x32_bf16 for the tile's 16 gate rows and one for its 16
                                    up rows, the E2M1 weights times their E8M0 block scale converted
                                    exactly to bf16, times the exact bf16 values of the E4M3 input codes,
                                    fp32 accumulation (within 2.7 * 2^-24 * sum |terms| per instruction,
                                    measured).  moe_decode_set_layer repacks the gate/up weights into that
                                    instruction's operand layout (same bytes per layer).  Without it the
                                    VALU form converts both to f16 and uses dot products.  The W4A8
                                    product (tanhow.com, section "为什么 DGX Spark 上的 MoE 解码是内存受限
                                    的"; devotd.net, section 2) is the same in both; measured on the
                                    42-layer stack it is faster at 4 tokens (the verify step) and slower at
                                    1, so it is a choice per handle, not the default. */
#define MOE_F_GENERIC 0x20u      /* use the shape-generic ahead-of-time kernels, which read the layer shape
                                    from their arguments.  Without it, a handle whose shape is the MoE
                                    layer of the pages' model (hidden 2560, 512 routed experts, top-8, 1
                                    shared, width 768: tanhow.com, section "Ling 3.0 是什么") runs a build
                                    of the same kernels with that shape folded in at compile time (as
                                    MOE_F_JIT does at run time), which computes the same results.  No
                                    effect with MOE_F_JIT. */

typedef struct moe_decode_handle moe_decode_handle;
typedef struct fp8_head_handle fp8_head_handle;

typedef struct {
    uint32_t struct_size; /* sizeof(moe_decode_config) */
    int32_t hidden;       /* H: multiple of 256, 256..2560 (the library checks that it has a kernel) */
    int32_t num_experts;  /* E routed experts: a multiple of 8 up to 512 */
    int32_t top_k;        /* k: 1..8, <= E */
    int32_t num_shared;   /* S: 0 or 1; the shared expert is stored at expert index E */
    int32_t inter;        /* I: SwiGLU width: 64, 128, 256 or 768 */
    int32_t max_tokens;   /* 1..4 tokens per run */
    int32_t num_layers;   /* L >= 1 */
    uint32_t flags;       /* MOE_F_* */
} moe_decode_config;

typedef struct {
    const void* ptr; /* device pointer */
    int32_t dtype;   /* moe_dtype tag; checked against the slot it is passed in */
} moe_tensor;

/* One layer's weights in canonical (row-major) layout.  set_layer copies and repacks them into
 * handle-owned device memory; the caller may free them once the stream has passed set_layer. */
typedef struct {
    moe_tensor router; /* BF16   [E][H] */
    moe_tensor w13;    /* E2M1X2 [E+S][2I][H/2]   rows 0..I-1 gate, rows I..2I-1 up */
    moe_tensor w13_s;  /* E8M0   [E+S][2I][H/32] */
    moe_tensor w2;     /* E2M1X2 [E+S][H][I/2]    down projection */
    moe_tensor w2_s;   /* E8M0   [E+S][H][I/32] */
} moe_layer_desc;

/* Outputs of one run; every pointer is a device pointer and may be NULL (not written). */
typedef struct {
    uint32_t struct_size;  /* sizeof(moe_outputs) */
    void* x_out;           /* BF16 [T][H]: residual after the last layer, x_L */
    float* y;              /* FP32 [T][H]: MoE output y of the last layer */
    int32_t* topk_ids;     /* [L][T][k]: expert ids, logit descending, lower index first on ties */
    float* topk_w;         /* [L][T][k]: softmax weights of the selected experts */
    void* x_trace;         /* BF16 [L][T][H]: each layer's input residual x_l */
    float* x_scale;        /* FP32 [L][T]: per-token activation scale s_x of each layer */
    uint8_t* x_codes;      /* E4M3 [L][T][H]: the quantised activation of each layer (8-byte aligned) */
} moe_outputs;

typedef struct {
    uint32_t struct_size;         /* sizeof(moe_decode_info) */
    char variant[64];             /* name of the kernel set in use */
    uint64_t weight_bytes;        /* handle-owned repacked weight memory, all layers */
    uint64_t workspace_bytes;     /* handle-owned scratch memory */
    uint64_t bytes_per_layer_t1;  /* algorithmic HBM bytes of one layer, 1 token */
    int32_t layers_set;           /* number of layers set so far */
    int32_t jit_from_cache;       /* MOE_F_JIT: 1 if the kernels were loaded from the cache, 0 if compiled */
    double jit_compile_ms;        /* MOE_F_JIT: hipRTC compile time at create (0 on a cache hit) */
    char jit_code_object[512];    /* MOE_F_JIT: path of the cached code object; "" otherwise */
} moe_decode_info;

/* Creates a handle bound to the current device: allocates repacked weight storage for all layers
 * and the workspace.  Returns MOE_ERR_NO_DEVICE when no HIP device is visible.  *out is written
 * only on success. */
moe_status moe_decode_create(const moe_decode_config* cfg, void* stream, moe_decode_handle** out);

/* Copies the weights of layer `layer` (0-based) into the handle, on `stream`, repacked into lane
 * tiles (a permutation of 16-byte units and scale bytes; no value changes). */
moe_status moe_decode_set_layer(moe_decode_handle* h, int32_t layer, const moe_layer_desc* desc, void* stream);

/* Runs all L layers on x (BF16 [T][H], device, 16-byte aligned), 1 <= T <= max_tokens.
 * Every layer must have been set.  Only enqueues work on `stream`.  By default, unless
 * MOE_F_DIRECT_LAUNCH is set, the first call with a given (x, T, outputs) captures the kernel
 * sequence (three kernels per layer, plus two small ones per layer at 3-4 tokens) into a HIP graph
 * owned by the handle and every later call with the same arguments replays it (up to 16 graphs;
 * they hold pointers, not data, so new contents of x and new weights are picked up).  A call with a
 * 17th set of arguments waits for the device to finish its queued work (hipDeviceSynchronize),
 * then drops the 16 graphs and captures anew; so does moe_decode_timing_enable. */
moe_status moe_decode_run(moe_decode_handle* h, const void* x, int32_t num_tokens, const moe_outputs* out,
                          void* stream);

moe_status moe_decode_query(const moe_decode_handle* h, moe_decode_info* info);

/* Waits for the handle's device to finish all work and returns MOE_ERR_HIP, with the runtime's
 * message in moe_last_error(), when that work ended in an asynchronous error; MOE_OK otherwise. */
moe_status moe_decode_check(moe_decode_handle* h);

/* Frees the handle's device memory (synchronises the device first).  NULL is a no-op. */
moe_status moe_decode_destroy(moe_decode_handle* h);

/* FP8 LM head (tanhow.com, section "三项优化是什么", item 2): logits[t][v] = s_v * sum_c W[v][c] x[t][c]
 * with W E4M3 [V][H] (row-major), s FP32 [V] per-row scales, x BF16 [T][H]; argmax[t] is the
 * lowest index among the maxima.  create copies W and s into handle-owned memory. */
moe_status fp8_head_create(int32_t vocab, int32_t hidden, moe_tensor w, moe_tensor row_scale, void* stream,
                           fp8_head_handle** out);
/* The unquantised head that the FP8 head replaces, for measuring what FP8 saves: W BF16 [V][H]
 * (row-major; no scales), otherwise as fp8_head_create.  The handle is run and freed with
 * fp8_head_run / fp8_head_destroy, which then compute logits[t][v] = sum_c W[v][c] x[t][c] (bf16
 * products, exact in fp32; fp32 accumulation) and the lowest-index argmax. */
moe_status bf16_head_create(int32_t vocab, int32_t hidden, moe_tensor w, void* stream, fp8_head_handle** out);
/* logits (FP32 [T][V], device) may be NULL; argmax (INT32 [T], device) is required. */
moe_status fp8_head_run(fp8_head_handle* h, const void* x, int32_t num_tokens, float* logits, int32_t* argmax,
                        void* stream);
moe_status fp8_head_destroy(fp8_head_handle* h);

/* The head of a speculative verify step with its greedy acceptance fused in (tanhow.com, section
 * "三项优化是什么", item 3: one verify pass scores the current token and the drafted ones;
 * devotd.net, "dgx-spark-moe-inference-optimizations", section 3).  x holds the T positions (BF16
 * [T][H], 2 <= T <= 4): the current token, then the T-1 drafted ones; draft (INT32 [T-1], device)
 * holds those drafted token ids.  Writes argmax[t] (INT32 [T]) as fp8_head_run does, and
 * accept[0] = the number n of leading drafts that equal the target's tokens (draft[i] ==
 * argmax[i] for every i < n, 0 <= n <= T-1); the step then emits draft[0 .. n-1] and argmax[n].
 * All pointers are device pointers; only enqueues work on `stream`. */
moe_status fp8_head_verify(fp8_head_handle* h, const void* x, int32_t num_tokens, const int32_t* draft,
                           int32_t* argmax, int32_t* accept, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the computation of fp8_head_run on the caller's own row-major
 * weights, with no handle.  w: E4M3 [vocab][hidden] row-major (16-byte aligned); row_scale: FP32
 * [vocab]; x, logits (nullable), argmax and num_tokens as in fp8_head_run.  Allocates nothing: the
 * argmax reduction's scratch (an arrival counter and per-workgroup maxima, 131,328 bytes) is one fixed
 * device array per GPU, held until the process ends; every call on a GPU uses that GPU's copy, so
 * calls that overlap on one GPU (other streams, other threads) race and must be serialised by the
 * caller.  The last workgroup of each call resets the counter to zero.  vocab above
 * MOE_NOALLOC_MAX_VOCAB returns MOE_ERR_INVALID_ARG; other errors as fp8_head_run.  Only enqueues
 * work on `stream`. */
#define MOE_NOALLOC_MAX_VOCAB 262144
moe_status fp8_head_run_noalloc(int32_t vocab, int32_t hidden, moe_tensor w, moe_tensor row_scale, const void* x,
                                int32_t num_tokens, float* logits, int32_t* argmax, void* stream);

/* Per-row FP8 quantisation of an LM-head weight matrix at load time, the step that makes the FP8
 * head (tanhow.com, section "三项优化是什么", item 2: the head is kept in FP8 instead of BF16 so that
 * each decode step reads half the bytes; devotd.net, "dgx-spark-moe-inference-optimizations",
 * section 2).  For every row r of W (BF16 or FP32 [rows][cols], row-major, tag checked):
 *   scales[r]   = fl32(max_c |W[r][c]| / 448), or 1 for an all-zero row;
 *   codes[r][c] = OCP E4M3 round-to-nearest-even of fl32(W[r][c] / scales[r]) (a NaN element gives
 *                 the NaN code S.1111.111 with its sign; NaNs do not enter the row maximum).
 * The outputs (E4M3 [rows][cols] and FP32 [rows], caller-owned device buffers, 8- and 4-byte
 * aligned) are the inputs fp8_head_create takes.  cols: a multiple of 256 up to 2560.  Only
 * enqueues work on `stream`; W may be freed after the stream has synchronised.  Errors:
 * MOE_ERR_INVALID_ARG (sizes, NULL or misaligned pointers), MOE_ERR_UNSUPPORTED (cols),
 * MOE_ERR_DTYPE (tag), MOE_ERR_NO_DEVICE, MOE_ERR_HIP (launch). */
moe_status fp8_head_quantize(int32_t rows, int32_t cols, moe_tensor w, void* codes, float* scales, void* stream);

/* Measurement probe: reads `bytes` (a multiple of 16) of device memory at src (16-byte aligned)
 * with the weight kernels' 16-byte non-temporal loads, `grid` workgroups of 256 threads, and writes
 * one fold of the data per workgroup to out (UINT32 [grid], device).  Timing it gives the practical
 * HBM read ceiling of that access pattern, reported beside the 8 TB/s peak.  Only enqueues work. */
moe_status moe_probe_stream_read(const void* src, uint64_t bytes, uint32_t* out, int32_t grid, void* stream);

/* Kernel timing instrumentation, for a measurement pass of its own.  moe_decode_timing_enable(h,
 * max_runs, mode) records the next up to max_runs calls of moe_decode_run; max_runs 0 disables.
 *   mode 0: the kernels are launched one by one on the caller's stream (no graph), each between a
 *           start and a stop HIP event that the runtime stamps with that kernel's own begin and end
 *           (hipExtLaunchKernel); total_ms[c] sums those durations.
 *   mode 1: the pass is replayed from a HIP graph as in normal runs, and every workgroup of every
 *           kernel writes the device's constant-rate wall clock at its start and end into a record
 *           that the library allocates at enable; each run waits for its pass and reduces the
 *           record: total_ms[c] sums, per kernel, the span from its first workgroup's start to its
 *           last workgroup's end, gap_ms[c] the time from the previous kernel's end to its start (the
 *           first kernel of a pass has none).  Over a pass, spans and gaps add up to the pass time.
 *           The stamping kernels are separate ahead-of-time instances (also on a MOE_F_JIT handle):
 *           the kernels of normal runs carry no timing code.
 * moe_decode_timing_read waits for the recorded runs, returns per kernel class the number of
 * launches and the summed times, and clears the record. */
#define MOE_TIMING_CLASSES 5 /* 0 input (3-4 tokens), 1 router + top-k, 2 gate/up, 3 h requantisation
                                (3-4 tokens), 4 down + combine */
typedef struct {
    uint32_t struct_size;                     /* sizeof(moe_decode_timing) */
    int32_t runs;                             /* runs recorded */
    int32_t mode;                             /* the mode they were recorded in */
    uint64_t launches[MOE_TIMING_CLASSES];
    double total_ms[MOE_TIMING_CLASSES];
    uint64_t gap_launches[MOE_TIMING_CLASSES]; /* mode 1: launches with a previous kernel in the pass */
    double gap_ms[MOE_TIMING_CLASSES];         /* mode 1 */
} moe_decode_timing;
moe_status moe_decode_timing_enable(moe_decode_handle* h, int32_t max_runs, int32_t mode);
moe_status moe_decode_timing_read(moe_decode_handle* h, moe_decode_timing* out);

const char* moe_status_string(moe_status s);
/* Message of the last failed call made by this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
